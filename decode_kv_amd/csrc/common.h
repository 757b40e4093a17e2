// Internal device helpers shared by the CSA2 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;   // CDNA wavefront
constexpr int kDk = 64;     // index key / query width (bytes)

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T bitcast(const auto& x) {
    return __builtin_bit_cast(T, x);
}

// a * b + c with a, b < 2^24, as one v_mad_u32_u24 (left to itself the
// compiler forms a multiply per product and a three-input add per pair: one
// VALU instruction more for every two products of the scoring epilogue)
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t d;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Integer score of one 16-token group against up to 64 index heads, on the
// int8 matrix cores.  One v_mfma_i32_16x16x64_i8 per block of 16 heads:
//   A = q rows (M = head, K = key byte), B = key rows (K = key byte, N = token).
// Lane l supplies row/column (l & 15) and key bytes [16*(l>>4), +16) of both
// operands, so any hardware ordering of K is the same for A and B and the dot
// product is exact.  The 16x16 int32 result gives lane l the dot products of
// token (l & 15) with heads 16*mb + 4*(l>>4) + i, i = 0..3; the epilogue applies
// ReLU and the head weight.  Returned: lane l's partial sum over its heads,
// before the four lane rows (l >> 4) are added (reduce_rows4).
template <int NB>
__device__ __forceinline__ uint32_t score_partial16(const i32x4 (&qa)[NB],
                                                    const uint32_t (&wr)[NB][4], i32x4 keyop) {
    i32x4 acc[NB];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[mb], keyop, i32x4{0, 0, 0, 0}, 0, 0, 0);
    uint32_t part = 0;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = acc[mb][i] > 0 ? acc[mb][i] : 0;   // ReLU, < 2^21
            part = mad_u24(wr[mb][i], (uint32_t)r, part);     // weight <= 15
        }
    return part;
}

// Four 16-token groups at once: part[u] holds lane l's partial of group u
// (token l & 15, the heads of lane row l >> 4).  Returns, in lane (r, c) =
// (l >> 4, l & 15), the full score of token c of group r: two exchanges across
// the wave halves and one across neighbouring rows (v_permlane32_swap and
// v_permlane16_swap, no LDS), three adds.
__device__ __forceinline__ uint32_t reduce_rows4(const uint32_t (&part)[4]) {
    // halves: lanes 0-31 keep groups 0/1 and receive them from lanes 32-63,
    // lanes 32-63 keep groups 2/3
    const auto x02 = __builtin_amdgcn_permlane32_swap(part[0], part[2], false, false);
    const auto x13 = __builtin_amdgcn_permlane32_swap(part[1], part[3], false, false);
    const uint32_t s02 = x02[0] + x02[1];   // rows 0,1: group 0 | rows 2,3: group 2 (rows r, r^2)
    const uint32_t s13 = x13[0] + x13[1];   // rows 0,1: group 1 | rows 2,3: group 3
    // rows: even rows keep s02, odd rows keep s13, each adding its neighbour's
    const auto y = __builtin_amdgcn_permlane16_swap(s02, s13, false, false);
    return y[0] + y[1];
}

// Load the q operands and per-lane weights of one sequence's index query.
//   q: [H][64] int8 of this sequence, w: [H] int8.
template <int NB>
__device__ __forceinline__ void load_index_query(const int8_t* __restrict__ q,
                                                 const int8_t* __restrict__ w, int H,
                                                 i32x4 (&qa)[NB], uint32_t (&wr)[NB][4]) {
    const int l = lane_id();
    const int row = l & 15, grp = l >> 4;
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
        const int h = mb * 16 + row;
        if (h < H)
            qa[mb] = *reinterpret_cast<const i32x4*>(q + (size_t)h * kDk + grp * 16);
        else
            qa[mb] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = mb * 16 + grp * 4 + i;
            wr[mb][i] = hh < H ? (uint32_t)(uint8_t)w[hh] : 0u;
        }
    }
}

// Max / sum of one value over the four lane rows of a wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48): v_permlane32_swap then v_permlane16_swap exchange whole
// rows between registers, with no LDS round trip.
__device__ __forceinline__ float rows4_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Max / sum of one value over all 64 lanes, in every lane: within each row
// of 16 by DPP (lane swaps of 1 and 2 by quad permutes, then row rotations by
// 4 and 8), then across the four rows with the lane-row swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_mov<0x124>(x));   // row_ror:4
    x = fmaxf(x, dpp_mov<0x128>(x));   // row_ror:8
    return rows4_max(x);
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x124>(x);
    x += dpp_mov<0x128>(x);
    return rows4_sum(x);
}

// Inclusive prefix sum over the 64 lanes of a wave, in DPP: row shifts by 1,
// 2, 4 and 8 inside each row of 16 lanes (lanes shifted in from outside the
// row add 0), then lane 15 broadcast into rows 1 and 3 and lane 31 into rows
// 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return x;
}

// Exclusive prefix sum of one int per thread over a block of NT threads (in
// thread order); total gets the block sum.  s_tmp holds NT / 64 ints.  Every
// thread of the block must call it (two barriers).
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
    const int l = lane_id(), wv = threadIdx.x / kWave;
    const int x = wave_inclusive_scan(v);
    if (l == kWave - 1) s_tmp[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        const int c = s_tmp[i];
        if (i < wv) before += c;
        total += c;
    }
    __syncthreads();
    return before + x - v;
}

// Two exclusive prefix sums at once (a and b, thread order), with the block
// sums; the same two barriers as one scan.  s_tmp holds 2 * NT / 64 ints.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* s_tmp, int& pa, int& pb,
                                                      int& ta, int& tb) {
    constexpr int NW = NT / kWave;
    const int l = lane_id(), wv = threadIdx.x / kWave;
    const int xa = wave_inclusive_scan(a), xb = wave_inclusive_scan(b);
    if (l == kWave - 1) {
        s_tmp[wv] = xa;
        s_tmp[NW + wv] = xb;
    }
    __syncthreads();
    int ba = 0, bb = 0;
    ta = 0;
    tb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int ca = s_tmp[i], cb = s_tmp[NW + i];
        if (i < wv) {
            ba += ca;
            bb += cb;
        }
        ta += ca;
        tb += cb;
    }
    __syncthreads();
    pa = ba + xa - a;
    pb = bb + xb - b;
}

// Rank of this lane among the set lanes of a wave mask (lanes below it).
__device__ __forceinline__ int lane_rank64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Upper end of the sub-range [nlo, nlo + 2^sh) of a radix digit, clipped to
// hi; unsigned so that ranges ending at INT_MAX do not overflow.
__device__ __forceinline__ int sub_range_hi(int nlo, int sh, int hi) {
    return (int)min((unsigned)hi, (unsigned)nlo + ((1u << sh) - 1u));
}

// Last digits of a radix select.  [lo, hi] (0 <= lo <= hi) holds cnt entries,
// one per thread at most (x; a thread without one passes a value outside the
// range), and the need-th largest of them (1 <= need <= cnt) is wanted.  Each
// pass splits the range into at most 256 sub-ranges of equal width (the top 8
// bits of x - lo), counts them in LDS, and keeps the one holding the need-th
// largest, until the range is one value.  On return lo == hi is that value,
// need counts how many entries equal to it are taken, and cnt how many there
// are.  Block-uniform arguments; s_h (256 words) and s_res[0..2] are LDS the
// caller may reuse only after a barrier; at most 4 passes for 31-bit values.
__device__ __forceinline__ void narrow_to_value(int x, int& lo, int& hi, int& need, int& cnt,
                                                uint32_t* s_h, int* s_res) {
    const int tid = threadIdx.x;
    while (lo < hi) {
        const unsigned width_m1 = (unsigned)(hi - lo);
        const int bits = 32 - __clz(width_m1);
        const int sh = bits > 8 ? bits - 8 : 0;
        if (tid < 256) s_h[tid] = 0;
        __syncthreads();
        if (x >= lo && x <= hi) atomicAdd(&s_h[(unsigned)(x - lo) >> sh], 1u);
        __syncthreads();
        if (tid < kWave) {
            // lane l holds sub-ranges 255-4l .. 252-4l: lane 0 the highest
            uint32_t c[4];
            int sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[i] = s_h[255 - 4 * tid - i];
                sum += (int)c[i];
            }
            const int incl = wave_inclusive_scan(sum);
            int above = incl - sum;
            if (above < need && need <= incl) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (above + (int)c[i] >= need) {
                        s_res[0] = 255 - 4 * tid - i;
                        s_res[1] = above;
                        s_res[2] = (int)c[i];
                        break;
                    }
                    above += (int)c[i];
                }
            }
        }
        __syncthreads();
        const int d = s_res[0];
        need -= s_res[1];
        cnt = s_res[2];
        const int nlo = lo + (d << sh);
        hi = sub_range_hi(nlo, sh, hi);
        lo = nlo;
    }
}

}  // namespace csa2
