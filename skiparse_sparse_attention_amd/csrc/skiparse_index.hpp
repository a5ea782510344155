// Index arithmetic of the Skiparse permutation and of the 3D-RoPE layout,
// shared by the host API and the HIP kernels.
//
// Scopes (Open-Sora Plan documentation, "Skiparse Attention", Single Skip Mode
// and Group Skip Mode); inside a scope the tokens keep their original order:
//   Single Skip: token n is in scope n mod k, at in-scope position n div k.
//   Group Skip: adjacent tokens form groups of k and group j = n div k is in
//     scope j mod k; token n sits at in-scope position (n div k^2)*k + n mod k
//     (the scope's earlier whole groups, then its offset inside its own group).
// Positions (Wan 2.1 report, section 4.2.1): n = (t*H + h)*W + w.
// RoPE split: head_dim is divided 2:3:3 over t, h, w; every axis chunk is a
//   whole number of the 16 equal "RoPE chunks" of head_dim/16 elements, so the
//   rotate-half partner of chunk c is always another whole chunk.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SKIPARSE_HD __host__ __device__ __forceinline__
#else
#define SKIPARSE_HD inline
#endif

namespace skiparse {

enum { kSingle = 0, kGroup = 1 };

// Token index of in-scope position p of scope s.
SKIPARSE_HD int64_t scope_token(int64_t p, int64_t s, int64_t k, int mode) {
    if (mode == kSingle) return p * k + s;
    return (p / k) * k * k + s * k + (p % k);
}

// Scope and in-scope position of token n.
SKIPARSE_HD void token_scope(int64_t n, int64_t k, int mode, int64_t* s, int64_t* p) {
    if (mode == kSingle) {
        *s = n % k;
        *p = n / k;
    } else {
        *s = (n / k) % k;
        *p = (n / (k * k)) * k + n % k;
    }
}

// The rotate-half pairs of 3D RoPE expressed in RoPE chunks (16 per head_dim).
// t axis: chunks [0,4) (2 pairs), h axis: [4,10) (3 pairs), w axis: [10,16) (3 pairs).
struct RopePair {
    int c1;      // first-half chunk
    int c2;      // its rotate-half partner chunk
    int axis;    // 0 = t, 1 = h, 2 = w
    int jchunk;  // frequency index of the first element of c1, in chunks, inside its axis
};

SKIPARSE_HD RopePair rope_pair(int cp) {
    // cp in [0, 8)
    RopePair r;
    if (cp < 2) {
        r.c1 = cp; r.c2 = cp + 2; r.axis = 0; r.jchunk = cp;
    } else if (cp < 5) {
        r.c1 = 4 + (cp - 2); r.c2 = r.c1 + 3; r.axis = 1; r.jchunk = cp - 2;
    } else {
        r.c1 = 10 + (cp - 5); r.c2 = r.c1 + 3; r.axis = 2; r.jchunk = cp - 5;
    }
    return r;
}

// Number of (cos, sin) pairs of the per-axis RoPE tables for a T x H x W grid:
// axis a of size S_a contributes S_a * d_a/2 pairs (d_t/2 = D/8, d_h/2 = d_w/2 = 3D/16).
SKIPARSE_HD int64_t rope_table_pairs(int64_t T, int64_t H, int64_t W, int D) {
    return T * (D / 8) + H * (3 * D / 16) + W * (3 * D / 16);
}

}  // namespace skiparse
