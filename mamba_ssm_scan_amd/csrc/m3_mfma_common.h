// m3_mfma_common.h -- device helpers shared by the chunked prefill kernels
// (m3_prefill_mfma.hip, m3_prefill_ws4.hip): bf16 packing, the MFMA wrappers,
// rotations, cross-lane scans, chunk addressing, the mask coefficient and the
// state map of a stretch of tokens. Device code only, internal linkage.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

#include "m3_device.h"

namespace m3 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int N = 128;     // state rows
constexpr int P = 64;      // head dim
constexpr int K = 64;      // rotation pairs
constexpr int NS = N + 8;  // LDS row stride (bf16 elements) of B~, C~ and g^T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInv2Pi = 0.15915494309189535f;
constexpr double kInv2PiD = 0.15915494309189533577;

__device__ __forceinline__ floatx4 mfma32(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(u32x2 a, u32x2 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b),
                                                     c, 0, 0, 0);
}
// two floats -> packed bf16 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ float lo16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// (cos, sin) of 2 pi * rev
struct CS {
    float c, s;
};
__device__ __forceinline__ CS cs_rev(float om_rev, float T) {
    const float r = __builtin_amdgcn_fractf(om_rev * T);
    return CS{__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r)};
}
// one packed pair (b0, b1) turned by -Phi: (c b0 + s b1, c b1 - s b0)
__device__ __forceinline__ unsigned rot_pair(unsigned w, CS t) {
    const float b0 = lo16(w), b1 = hi16(w);
    return pack2(t.c * b0 + t.s * b1, t.c * b1 - t.s * b0);
}
// sum of the two products of packed bf16 pairs, in fp32
__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), 0.f, false);
}
// one packed bf16 pair (b0, b1) turned by -Phi, with cs = packed bf16 (cos Phi,
// sin Phi): (c b0 + s b1, c b1 - s b0), two dot products
__device__ __forceinline__ unsigned rot_cs(unsigned w, unsigned cs) {
    const unsigned ms_c = __builtin_amdgcn_perm(cs, cs, 0x01000302u) ^ 0x00008000u;  // (-s, c)
    return pack2(dot2_bf16(cs, w), dot2_bf16(ms_c, w));
}
// Transposing LDS load (ds_read_b64_tr_b16): in each group of 16 lanes, lane t
// gives the address of 4 consecutive 16-bit values of row t / 4 (columns
// 4 (t % 4) ..); lane j receives column j of those 4 rows. From a row-major
// [k][m] tile this yields the MFMA operand layout "lane = m, 4 consecutive k".
typedef short shortx4_tr __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 load_tr(const uint16_t* p) {
    const shortx4_tr v =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4_tr*)(p));
    return __builtin_bit_cast(u32x2, v);
}
// a packed bf16 pair times (wl, wh), repacked
__device__ __forceinline__ unsigned scale2(unsigned w, float wl, float wh) { return pack2(lo16(w) * wl, hi16(w) * wh); }
// broadcast lane j of every DPP quad
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), J * 0x55, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_read(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Inclusive prefix sum over the 64 lanes of a wavefront, kept off the LDS
// crossbar (a ds_bpermute shuffle would queue behind the MFMA operand reads and
// serialise every step): DPP right shifts inside each 16-lane row, then the
// row totals carried across rows through scalar registers.
__device__ __forceinline__ float wave_prefix_sum(float v, int lane) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
    const float r0 = lane_read(v, 15), r1 = lane_read(v, 31), r2 = lane_read(v, 47);
    const int row = lane >> 4;
    return v + ((row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f));
}
// value of lane 16 * (lane / 16) + 15 (the last lane of each row)
__device__ __forceinline__ float row_last(float v, int lane) {
    const float r0 = lane_read(v, 15), r1 = lane_read(v, 31), r2 = lane_read(v, 47), r3 = lane_read(v, 63);
    const int row = lane >> 4;
    return row == 0 ? r0 : row == 1 ? r1 : row == 2 ? r2 : r3;
}
// value of the last lane of each group of 16 / R lanes (lane = token: the last
// token whose rows fall in the same 16-row tile)
template <int LR>
__device__ __forceinline__ float tile_last(float v, int lane) {
    if constexpr (LR == 3) {  // two tokens per tile: lane 2k + 1 (DPP quad_perm [1, 1, 3, 3])
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xf5, 0xf, 0xf, false));
    } else if constexpr (LR == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xff, 0xf, 0xf, false));
    } else if constexpr (LR == 1) {
        const int q = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xff, 0xf, 0xf, false);  // lane 4k+3
        const int u = __builtin_amdgcn_update_dpp(q, q, 0x104, 0xf, 0xf, false);  // row_shl:4 -> lane 8k+7
        return __builtin_bit_cast(float, (lane & 4) ? q : u);
    } else {
        return row_last(v, lane);
    }
}

// Wait for this wave's LDS traffic, then meet the other waves. Unlike
// __syncthreads() this does not wait for outstanding global loads, so the next
// chunk's prefetch stays in flight across it.
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row addressing inside one chunk: token i, rank r of B/C sits at (i*G*R + r)*N
// elements past the chunk's first row, of x/y at (i*H*R + r)*P. Tokens past
// the chunk's end are clamped to its last token, so every load is
// unconditional and finite; such rows never reach a result: their mask
// entries and state weights are zero (their dt is taken as 0) and their
// outputs are not stored.
struct ChunkBase {
    const uint16_t* B;
    const uint16_t* C;
    const uint16_t* x;
    int nq;
    int nin;   // state rows this pass takes from the caller's B/C rows (<= N); rows nin..N-1 are zero
    int nrow;  // length of the caller's B/C rows (the caller's N)
    int pin;   // columns this pass takes from the caller's x rows (<= P); columns pin..P-1 are zero
    int pcol;  // length of the caller's x rows (the caller's P)
    int rin;   // the caller's rank (<= the kernel's R); ranks rin..R-1 are zero rows
};

// One pass of the chunked kernels over rows n_off .. n_off + nin - 1 of the
// caller's N (= nrow) and columns p_off .. p_off + pin - 1 of its P (= pcol).
// The state rows evolve independently and so do its columns: a column block
// is a problem of its own, a row block contributes a share of y that the
// passes sum in fp32 in ypart ([b][L][H][R][P]). ym: 0 the only row pass (y
// written in bf16), 1 first (writes ypart, with D x), 3 middle (adds to
// ypart), 2 last (adds ypart, writes y in bf16).
struct PassArgs {
    int nin, nrow, n_off, pin, pcol, p_off, ym;
    int rin;  // the caller's rank: R 3 runs on the R 4 kernel with a zero fourth rank
    float* ypart;
};

__device__ __forceinline__ u32x4 load_tok(const uint16_t* base, int i, int nq, int tok_stride, int off) {
    const int ic = i < nq ? i : nq - 1;
    return *reinterpret_cast<const u32x4*>(base + (ic * tok_stride + off));
}

// M_ij (decay x width-2 convolution mask) for row token tj and column token ti.
// Branch-free: the loads are always in range (tj < 64) and the causal cut is a
// select, so a wavefront whose lanes straddle the diagonal does not diverge.
__device__ __forceinline__ float mask_coef(int tj, int ti, float S2i, const float* w) {
    const float s2j = w[tj], gam = w[64 + tj], dln = w[128 + tj];
    const float coef = __builtin_amdgcn_exp2f(S2i - s2j) * (gam + (tj < ti ? dln : 0.f));
    return tj > ti ? 0.f : coef;
}

// Sequence segments (decoupled look-back). Workspace layout, per (b, h, segment)
// index bs = (b*H + h) * nseg + seg: ctrl[0] ticket counter, ctrl[1] error flag
// (a look-back wait that ran out of patience), ctrl[2 + bs] state flag
// (1 = local end state published, 2 = inclusive end state published);
// agg/incl [bs][N][P] fp32; tr[bs] the segment's total step (sum of dt).
struct SegArgs {
    int nseg;
    int64_t cps;  // chunks per segment
    unsigned* ctrl;
    float* agg;
    float* incl;
    double* tr;
    long spin_limit;  // polls before a look-back wait gives up (0: give up at once)
};

// The state map of a stretch with total step T: pair k turned by omega_k T and
// scaled by e^{A T}; om_rev = omega_k / 2 pi of the lane's two pairs.
__device__ __forceinline__ floatx4 transfer(floatx4 v, float A2, const float* om_rev, double T) {
    const float dec = __builtin_amdgcn_exp2f(float(double(A2) * T));
    floatx4 o;
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
        const double rv = double(om_rev[hp]) * T;
        const float r = float(rv - floor(rv));
        const float c = __builtin_amdgcn_cosf(r) * dec, sn = __builtin_amdgcn_sinf(r) * dec;
        o[2 * hp] = c * v[2 * hp] - sn * v[2 * hp + 1];
        o[2 * hp + 1] = sn * v[2 * hp] + c * v[2 * hp + 1];
    }
    return o;
}


}  // namespace
}  // namespace m3
