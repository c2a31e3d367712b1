// kvq_layout.h -- placement of a V code in the 32-token tiled layout used by
// the matrix-core attention kernel (host and device).
//
// A 32-token block of one stream holds the same number of words as 32
// token-major rows.  It is cut into 64 fragments, one per lane of the wave that
// consumes it: fragment f = 16*q + c16 feeds lane f of the P.V matrix product,
// i.e. channel row c16 of every 16-channel tile m, for the eight "k-slots"
// s = 0..7 that lane contributes, s < 4 -> token 4q+s, s >= 4 -> token
// 16+4q+(s-4).  Inside a fragment, 16-bit halves of consecutive words hold the
// (tile m, slot-pair) operand registers in order: register R = 4m + s/2,
// low half for even s, high half for odd s, P = 16 / vb registers per word.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

__host__ __device__ inline void v_tile_pos(int tb, int c, int vb, int D, int *word, int *bit)
{
    const int tile = tb >> 4, r16 = tb & 15, q = r16 >> 2, jj = r16 & 3;
    const int s = tile * 4 + jj;  // k-slot of this token
    const int m = c >> 4, c16 = c & 15;
    const int frag = q * 16 + c16;
    const int fw = D * vb / 64;  // words per fragment
    const int P = 16 / vb;       // registers (code pairs) per word
    const int R = 4 * m + (s >> 1);
    *word = frag * fw + R / P;
    *bit = vb * (R % P) + 16 * (s & 1);
}

}  // namespace kvq
