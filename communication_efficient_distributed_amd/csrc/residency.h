// residency.h -- cap on the workgroups a streaming kernel keeps on one CU.
//
// A launch may request dynamic LDS that the kernel never touches; the
// hardware then admits only as many of its workgroups per CU as fit in the
// CU's 160 KiB of LDS.  For kernels that read and write HBM in one pass, a CU
// full of workgroups keeps more requests in flight than the memory system
// serves well: reads and writes interleave more finely at the DRAM and the
// throughput drops (on MI355X a memory-only probe of the read 2 : write 1 mix
// ran 6.0 TB/s with 8 four-wavefront workgroups per CU and 6.4 TB/s with 2-3).
#pragma once

#include <stddef.h>

namespace sl {

constexpr int kLdsPerCu = 160 * 1024;

// LDS per workgroup that admits cap workgroups per CU and not cap + 1: whole
// KiB less a margin for the allocation granule.
constexpr size_t capped_workgroup_lds(int cap) { return (size_t)(kLdsPerCu / cap / 1024) * 1024 - 64; }

constexpr bool cap_is_exact(int cap, size_t static_lds) {
    return cap * capped_workgroup_lds(cap) <= (size_t)kLdsPerCu &&
           (cap + 1) * capped_workgroup_lds(cap) > (size_t)kLdsPerCu && capped_workgroup_lds(cap) >= static_lds;
}

// Dynamic LDS bytes to request for a kernel with static_lds bytes of its own.
constexpr size_t residency_lds(int cap, size_t static_lds) { return capped_workgroup_lds(cap) - static_lds; }

}  // namespace sl
