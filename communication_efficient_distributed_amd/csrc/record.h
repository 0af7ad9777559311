// record.h -- device-side reading of the 112-byte chunk record written by the
// compressor: 64 12-bit indices (bytes 0..95) then 64 2-bit codes (bytes
// 96..111), both little-endian LSB-first bit streams (layout documented with
// sl_compress in include/sparseloco.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparseloco.h"

namespace sl {

// Entry j of a record: its 12-bit index sits in the 3-byte group of the pair
// (j & ~1, j | 1) at byte 3*(j >> 1), low half for even j; its 2-bit code is
// field (j & 15) of code word 24 + (j >> 4).
struct EntryPos {
    int w0, sh, cw, csh;
    __device__ explicit EntryPos(int j) {
        const int grp = 3 * (j >> 1);
        w0 = grp >> 2;
        sh = (grp & 3) * 8 + ((j & 1) ? 12 : 0);
        cw = SL_INDEX_BYTES / 4 + (j >> 4);
        csh = 2 * (j & 15);
    }
    // index | code << 12 of entry j of the record whose dwords start at rec
    __device__ __forceinline__ uint32_t read(const uint32_t* rec) const {
        const uint32_t a = rec[w0], b = rec[w0 + 1], c = rec[cw];
        const uint32_t idx = (uint32_t)((((uint64_t)b << 32) | a) >> sh) & 4095u;
        return idx | (((c >> csh) & 3u) << 12);
    }
};

}  // namespace sl
