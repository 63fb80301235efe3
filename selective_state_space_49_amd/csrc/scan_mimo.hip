// scan_mimo.hip -- prefill with multi-input multi-output (MIMO) projections (gfx950).
//
// The Mamba-3 item on MIMO ("Jamba — SSM-Transformer Híbrido", section "Mamba-3: a
// linha de base de SSM puro em 2026", item 3) makes the per-feature projections
// matrix-valued. Read here as: each channel takes R inputs and gives R outputs, and
// B_t, C_t are N x R matrices shared by the channels of a (batch, step):
//     h_t[n] = exp(dt_t A[n]) h_{t-1}[n] + dt_t sum_r B_t[n][r] x_t[r]
//     y_t[r] = (sum_n C_t[n][r] h_t[n] + D x_t[r]) * silu(z_t[r])
// The state stays N wide per channel; R = 1 is the plain scan.
//
// Work split and phases are those of the plain prefill: one lane per channel with its
// N states in VGPRs, the sequence cut into chunks (summary from a zero start over the
// decay window, carry scan over chunks, rescan with the epilogue). The decay of a step
// does not depend on R, so the decay horizon and the carry kernel are shared as they
// are. What changes is the per-step work: the R inputs of a channel are one vector
// load (R consecutive elements of a [rows][Dn][R] stream), B_t and C_t come in through
// the scalar unit as N*R wave-uniform values, and each state update costs R
// multiply-adds for B_t x_t and each output R more for C_t h_t, against one
// exponential per state: the exponential is shared by R outputs.
//
// From rank 4 the rescan and the summaries compute B_t x_t on the matrix cores, with
// B_t's rows staged through LDS (mimo_bx, mimo_steps); with bf16 inputs the rescan also
// takes the outputs' sums over the states, sum_n C_t[n][r] h[n], there, with C_t's rows
// staged through LDS transposed (mimo_update, CStage). The decode step (k_mimo_step) advances one token per (layer,
// sequence, channel) with the VALU form of the same step function.
#include "ssm_device.h"
#include "ssm_internal.h"
#include "ssm_stream.h"

namespace ssm {
namespace {

typedef uint32_t u32x2 __attribute__((vector_size(8)));
typedef uint32_t u32x4 __attribute__((vector_size(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a and b rounded to bf16 (to nearest even) and packed, a in the low half: one
// v_cvt_pk_bf16_f32 (two scalar conversions would each take one, plus a shift and an or).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// The R elements of one channel in one row, as loaded (raw bits).
template <typename IO, int R>
struct VecRaw {
    static constexpr int kBytes = R * (int)sizeof(IO);
    static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
    uint32_t w[kWords];
    // Element r, widened to fp32 (exact).
    __device__ __forceinline__ float at(int r) const {
        if constexpr (sizeof(IO) == 2) {
            const uint32_t v = w[r >> 1];
            return __uint_as_float((r & 1) ? (v & 0xffff0000u) : (v << 16));
        } else {
            return __uint_as_float(w[r]);
        }
    }
};

// A [rows][Dn][R] stream walked row by row through a buffer resource, like RowStream:
// voff = the lane's channel times R elements, soff = the row's byte offset.
template <typename IO, int R>
struct VecStream {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit VecStream(const void *base)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, -1, kRsrcWord3)) {}

    __device__ __forceinline__ VecRaw<IO, R> ld(uint32_t voff, uint32_t soff) const {
        VecRaw<IO, R> v;
        constexpr int B = VecRaw<IO, R>::kBytes;
        if constexpr (B == 2) {
            v.w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
        } else if constexpr (B == 4) {
            v.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        } else if constexpr (B == 8) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
            v.w[0] = t[0]; v.w[1] = t[1];
        } else if constexpr (B == 16) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) v.w[k] = t[k];
        } else {
            static_assert(B == 32, "R * element size must be 2..32 bytes");
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16u * h, soff, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) v.w[4 * h + k] = t[k];
            }
        }
        return v;
    }

    // Stores y[0..R) (rounded to the element type) with one vector store, streaming
    // (glc slc): y is written once and read only by the caller's next step.
    __device__ __forceinline__ void st(uint32_t voff, uint32_t soff, const float (&y)[R]) const {
        VecRaw<IO, R> v;
        if constexpr (sizeof(IO) == 2) {
            if constexpr (R == 1) {
                v.w[0] = f32_to_bf16(y[0]);
            } else {
#pragma unroll
                for (int k = 0; k < R / 2; ++k)
                    v.w[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < R; ++k) v.w[k] = __float_as_uint(y[k]);
        }
        constexpr int B = VecRaw<IO, R>::kBytes;
        if constexpr (B == 2) {
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v.w[0], r, voff, soff, 3);
        } else if constexpr (B == 4) {
            __builtin_amdgcn_raw_buffer_store_b32(v.w[0], r, voff, soff, 3);
        } else if constexpr (B == 8) {
            u32x2 t = {v.w[0], v.w[1]};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, voff, soff, 3);
        } else if constexpr (B == 16) {
            u32x4 t = {v.w[0], v.w[1], v.w[2], v.w[3]};
            __builtin_amdgcn_raw_buffer_store_b128(t, r, voff, soff, 3);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                u32x4 t = {v.w[4 * h], v.w[4 * h + 1], v.w[4 * h + 2], v.w[4 * h + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(t, r, voff + 16u * h, soff, 3);
            }
        }
    }
};

// R consecutive elements at a global pointer (aligned to min(16, R * element) bytes).
template <typename IO, int R>
__device__ __forceinline__ VecRaw<IO, R> ld_vec(const IO *p) {
    VecRaw<IO, R> v;
    constexpr int B = VecRaw<IO, R>::kBytes;
    if constexpr (B == 2) {
        v.w[0] = *(const uint16_t *)p;
    } else if constexpr (B == 4) {
        v.w[0] = *(const uint32_t *)p;
    } else if constexpr (B == 8) {
        const u32x2 t = *(const u32x2 *)p;
        v.w[0] = t[0]; v.w[1] = t[1];
    } else {
#pragma unroll
        for (int h = 0; h < B / 16; ++h) {
            const u32x4 t = *((const u32x4 *)p + h);
#pragma unroll
            for (int k = 0; k < 4; ++k) v.w[4 * h + k] = t[k];
        }
    }
    return v;
}

// Stores y[0..R), rounded to the element type, with one vector store (two for 32 bytes).
template <typename IO, int R>
__device__ __forceinline__ void st_vec(IO *p, const float (&y)[R]) {
    VecRaw<IO, R> v;
    if constexpr (sizeof(IO) == 2) {
        if constexpr (R == 1) {
            *(uint16_t *)p = f32_to_bf16(y[0]);
            return;
        } else {
#pragma unroll
            for (int k = 0; k < R / 2; ++k)
                v.w[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
        }
    } else {
#pragma unroll
        for (int k = 0; k < R; ++k) v.w[k] = __float_as_uint(y[k]);
    }
    constexpr int B = VecRaw<IO, R>::kBytes;
    if constexpr (B == 4) {
        *(uint32_t *)p = v.w[0];
    } else if constexpr (B == 8) {
        const u32x2 t = {v.w[0], v.w[1]};
        *(u32x2 *)p = t;
    } else {
#pragma unroll
        for (int h = 0; h < B / 16; ++h) {
            const u32x4 t = {v.w[4 * h], v.w[4 * h + 1], v.w[4 * h + 2], v.w[4 * h + 3]};
            *((u32x4 *)p + h) = t;
        }
    }
}

// Ranks 4 and 8 compute B_t x_t on the matrix cores; ranks 1 and 2 on the VALU, rank 1
// with exactly the plain scan's operations (rank 2 measured faster on the VALU).
template <int R> constexpr bool kMatInput = R >= 4;

// The input term of state n at row element e = e0 + n R (VALU path): u = sum_r B[n][r]
// xd[r] with xd = dt x, as u = B[n][0] xd[0], then u = fma(B[n][r], xd[r], u).
template <int R, typename Row>
__device__ __forceinline__ float mimo_input(const Row &Bp, int64_t e, const float (&xd)[R]) {
    float u = Bp.ld(e) * xd[0];
#pragma unroll
    for (int r = 1; r < R; ++r) u = __builtin_fmaf(Bp.ld(e + r), xd[r], u);
    return u;
}

// B_t x_t on the matrix cores (ranks 4 and 8): v[n] = sum_r B_t[n][r] x[r] for all N
// states of every lane's channel. For each group of four states n0 .. n0+3, bf16 takes
// one v_mfma_f32_4x4x4_16b_bf16 per 4 ranks and fp32 one v_mfma_f32_4x4x1_16b_f32 per
// rank: lane l supplies row n0 + l%4 of B_t as the A operand and its own x as the B
// operand, and the 16-block 4x4 forms give D[l][i] = sum_k A[4 (l/4) + i][k] B[l][k]
// (a layout a probe confirmed), so result register i of lane l is v[n0 + i] of lane
// l's channel: the layout the state is kept in. Products of bf16 values are exact in
// fp32. Every lane of the wave takes part (a block reads the A operand of all four of
// its lanes), so the kernels keep lanes past the last channel running on clamped
// indices. brow: the step's B row ([N][R], 16-byte aligned), in LDS or global memory.
typedef short s4v __attribute__((ext_vector_type(4)));
typedef float f4m __attribute__((ext_vector_type(4)));
#define SSM_LDS __attribute__((address_space(3)))

// A T at byte pointer p, in global memory or in LDS.
template <typename T> __device__ __forceinline__ T ld_at(const char *p) { return *(const T *)p; }
template <typename T> __device__ __forceinline__ T ld_at(const SSM_LDS char *p) {
    return *(const SSM_LDS T *)p;
}

__device__ __forceinline__ f4m mma_bf16(u32x2 a, u32x2 b, f4m c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s4v, a), __builtin_bit_cast(s4v, b),
                                                  c, 0, 0, 0);
}

// v[n0 + i] (i = 0..3) for the group of states n0 = 4 g (mimo_bx_group), or for all N.
template <typename IO, int N, int R, typename P>
__device__ __forceinline__ f4m mimo_bx_group(P brow, const VecRaw<IO, R> &xr, int g) {
    static_assert(R == 4 || R == 8, "matrix path: ranks 4 and 8");
    // N < 4: rows past the last state only fill result registers that are not used
    const uint32_t n = min(4u * g + (threadIdx.x & 3u), (uint32_t)N - 1u);
    const P p = brow + n * (uint32_t)(R * sizeof(IO));
    f4m d = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (sizeof(IO) == 2) {
#pragma unroll
        for (int k = 0; k < R / 4; ++k) {
            const u32x2 av = ld_at<u32x2>(p + 8 * k);
            const u32x2 bv = {xr.w[2 * k], xr.w[2 * k + 1]};
            d = mma_bf16(av, bv, d);
        }
    } else {
#pragma unroll
        for (int k = 0; k < R / 4; ++k) {
            const u32x4 t = ld_at<u32x4>(p + 16 * k);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                d = __builtin_amdgcn_mfma_f32_4x4x1f32(__uint_as_float(t[j]), xr.at(4 * k + j), d, 0, 0, 0);
        }
    }
    return d;
}

template <typename IO, int N, int R, typename P>
__device__ __forceinline__ void mimo_bx(P brow, const VecRaw<IO, R> &xr, float (&v)[N]) {
#pragma unroll
    for (int g = 0; g < (N + 3) / 4; ++g) {
        const f4m d = mimo_bx_group<IO, N, R>(brow, xr, g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i < N) v[4 * g + i] = d[i];
    }
}

// Outputs on the matrix cores: bf16 inputs from rank 4, at least 4 states (fp32 inputs
// keep the exact VALU sums: the fp32 matrix form, one v_mfma_f32_4x4x1_16b_f32 per state
// and four ranks, measured no faster than the multiply-adds it replaces).
template <typename IO, int N, int R>
constexpr bool kMatOutput = kMatInput<R> && sizeof(IO) == 2 && N >= 4;

// The A operands of the matrix outputs for one step: quad(n0, g) = the bf16 values
// C_t[n0 + k][4g + l%4], k = 0..3, of lane l, packed two to a word. COpsLds reads them
// from the wave's C slot (CStage), COpsGlb from the step's C row in global memory (the
// ragged tail), CNone stands in where the outputs are not on the matrix cores.
template <int N>
struct COpsLds {
    const SSM_LDS uint16_t *p;  // the lane's rank-(l%4) row of the step, [R][N] layout
    __device__ __forceinline__ u32x2 quad(int n0, int g) const {
        return *(const SSM_LDS u32x2 *)(p + 4 * g * N + n0);
    }
};
template <int N, int R>
struct COpsGlb {
    const uint16_t *p;  // the step's C row, [N][R]
    __device__ __forceinline__ u32x2 quad(int n0, int g) const {
        const uint16_t *c = p + n0 * R + 4 * g + (threadIdx.x & 3u);
        return u32x2{(uint32_t)c[0] | ((uint32_t)c[R] << 16), (uint32_t)c[2 * R] | ((uint32_t)c[3 * R] << 16)};
    }
};
struct CNone {};

// One step of one channel. The prefill rescan takes the matrix path from rank 4 (MAT),
// the decode step always the VALU path: it is bound by HBM, and the matrix operands'
// registers would cost it waves (65.3 against 58-60 us per call at rank 4). Up to rank 2
// the two therefore perform the same operations and L decode steps equal a one-chunk
// prefill bit for bit; from rank 4 they differ in the rounding of the sums.
// VALU path:  xd[r] = dt x[r];  for n ascending: h[n] = fma(e2(dt A[n] log2 e), h[n],
//             mimo_input(n));  acc[r] = fma(C[n][r], h[n], acc[r])  (r ascending, acc
//             from 0). Bp / Cp read element e0 + n R + r of the step's B / C through the
//             scalar unit.
// Matrix path: v = B_t x_t (mimo_bx_group, four states at a time; brow the step's B
//             row);  for n ascending: h[n] = fma(e2(dt A[n] log2 e), h[n], dt v[n]).
//             Outputs with bf16 inputs (kMatOutput): after each group of four states
//             n0 .. n0+3, acc[4g .. 4g+3] += sum_k C_t[n0+k][4g+i] h[n0+k] by one
//             v_mfma_f32_4x4x4_16b_bf16 per group g of four ranks: lane m supplies
//             C_t[n0+k][4g + m%4] (cops, bf16 and exact) as the A operand and lane l its
//             own h[n0+k] rounded to bf16 as the B operand, so result register i of lane
//             l is rank 4g + i of lane l's channel (the layout of mimo_bx). The state
//             itself stays fp32; only its copy in the output sum is rounded, which adds
//             at most 2^-8 sum_n |C[n][r] h[n]| to y[r], the size of y's own rounding
//             to bf16 on the way out. Otherwise acc[r] = fma(C[n][r], h[n], acc[r]) as
//             on the VALU path.
template <typename IO, int N, int R, bool MAT, typename Row, typename P, typename COps>
__device__ __forceinline__ void mimo_update(float (&h)[N], const float (&A2)[N], float dv,
                                            const VecRaw<IO, R> &xr, const float (&xv)[R],
                                            const Row &Bp, const Row &Cp, P brow, const COps &cops,
                                            int64_t e0, float (&acc)[R]) {
    if constexpr (MAT) {
        // group by group of four states, so that only four input terms are live
        constexpr bool kOut = kMatOutput<IO, N, R>;
        f4m d[R / 4];
#pragma unroll
        for (int g = 0; g < R / 4; ++g) d[g] = f4m{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int q = 0; q < (N + 3) / 4; ++q) {
            const f4m v = mimo_bx_group<IO, N, R>(brow, xr, q);
#pragma unroll
            for (int i = 0; i < 4 && 4 * q + i < N; ++i) {
                const int n = 4 * q + i;
                h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], dv * v[i]);
                if constexpr (!kOut) {
                    const int64_t e = e0 + n * R;
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(Cp.ld(e + r), h[n], acc[r]);
                }
            }
            if constexpr (kOut) {
                const u32x2 hp = {pack_bf16x2(h[4 * q], h[4 * q + 1]), pack_bf16x2(h[4 * q + 2], h[4 * q + 3])};
#pragma unroll
                for (int g = 0; g < R / 4; ++g) d[g] = mma_bf16(cops.quad(4 * q, g), hp, d[g]);
            }
        }
        if constexpr (kOut) {
#pragma unroll
            for (int g = 0; g < R / 4; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[4 * g + i] = d[g][i];
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
        float xd[R];
#pragma unroll
        for (int r = 0; r < R; ++r) xd[r] = dv * xv[r];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            const int64_t e = e0 + n * R;
            h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], mimo_input<R>(Bp, e, xd));
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(Cp.ld(e + r), h[n], acc[r]);
        }
    }
}

// y[r] = fma(D, x[r], acc[r]), gated: y[r] * silu(z[r]).
template <typename IO, int R, bool GATED>
__device__ __forceinline__ void mimo_out(float Dd, const float (&xv)[R], const float (&acc)[R],
                                         const VecRaw<IO, R> &zr, float (&yv)[R]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        yv[r] = __builtin_fmaf(Dd, xv[r], acc[r]);
        if (GATED) yv[r] = yv[r] * silu(zr.at(r));
    }
}

// One block of KU steps of loaded inputs (raw bits, widened at use), and the lane's
// CW words of the block's C rows when the outputs are on the matrix cores.
template <typename IO, int R, int KU, int CW>
struct MimoBlock {
    VecRaw<IO, R> x[KU], z[KU];
    uint32_t dt[KU];
    uint32_t cw[CW];
};

struct MimoStreams {
    uint32_t vx;   // lane's byte offset in an x / z / y row
    uint32_t vd;   // lane's byte offset in a dt row
    uint32_t rbx;  // bytes per x / z / y row
    uint32_t rbd;  // bytes per dt row
};

template <typename IO, int R, bool GATED, int KU, int CW>
__device__ __forceinline__ void load_mimo_block(MimoBlock<IO, R, KU, CW> &s, const VecStream<IO, R> &x,
                                                const RowStream<IO> &dt, const VecStream<IO, R> &z,
                                                const MimoStreams &o, uint32_t row) {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
        s.x[k] = x.ld(o.vx, (row + k) * o.rbx);
        s.dt[k] = dt.ldraw(o.vd, (row + k) * o.rbd);
        if (GATED) s.z[k] = z.ld(o.vx, (row + k) * o.rbx);
    }
}

// s_waitcnt for the vector-memory counter only (lgkmcnt and expcnt left at their
// maxima), and for the LDS / scalar counter only.
__device__ __forceinline__ constexpr int wait_vm(int n) {
    return (n & 0xF) | ((n >> 4) & 0x3) << 14 | 0x70 | 0xF00;
}
constexpr int kWaitLgkm0 = 0xC07F;

// Staging of B_t rows for the matrix path. Each wave owns a ring of two slots of KU
// rows in LDS; the rows of the next block are copied in by direct-to-LDS buffer loads
// (4 bytes per lane, so 256 bytes per instruction, no registers held while in flight)
// together with that block's x, dt and z, while the current block is computed. The
// compiler does not order these loads against LDS reads, so the loop waits itself:
//   - before a slot is refilled, lgkmcnt(0): the reads of the block that used it are done;
//   - before a block's rows are read, vmcnt(n) with n = the vector-memory instructions
//     issued for the next block just before: memory operations retire in order, so
//     everything older, this block's staging loads among it, is then complete.
template <typename IO, int N, int R, int KU>
struct BStage {
    static constexpr int kRowBytes = N * R * (int)sizeof(IO);
    static constexpr int kSlotBytes = KU * kRowBytes;
    static constexpr int kLoads = (kSlotBytes + 255) / 256;            // per slot
    static constexpr int kLastLanes = (kSlotBytes - 256 * (kLoads - 1)) / 4;
    __amdgpu_buffer_rsrc_t r;  // this walk's B rows, from its first row on
    SSM_LDS char *ring;        // 2 slots of kSlotBytes
    __device__ __forceinline__ void stage(int slot, uint32_t row) const {
        const uint32_t lane = threadIdx.x & 63u;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
        for (int d = 0; d < kLoads; ++d) {
            if (d < kLoads - 1 || lane < (uint32_t)kLastLanes)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SSM_LDS void *)(ring + slot * kSlotBytes + 256 * d), 4,
                                                         lane * 4u + 256u * d, row * (uint32_t)kRowBytes, 0, 0);
        }
    }
    __device__ __forceinline__ const SSM_LDS char *row_at(int slot, int j) const {
        return ring + slot * kSlotBytes + j * kRowBytes;
    }
};

// Staging of C_t rows for the matrix outputs (rescan; bf16, from rank 4). The block's C
// rows, [KU][N][R] elements and contiguous, are loaded into registers with the block's
// x, dt and z (kWords words per lane, one vector load). At the start of the block each
// lane writes its elements to the wave's slot in LDS transposed to [KU][R][N], so that
// the four operands lane l takes for rank r and states n0 .. n0+3 are one 8-byte read
// (the lanes of one rank read the same address: a broadcast). One slot suffices: a
// wave's LDS accesses complete in order, so a block's writes follow every read of the
// block before.
template <typename IO, int N, int R, int KU>
struct CStage {
    static constexpr int kRowBytes = N * R * (int)sizeof(IO);
    static constexpr int kBlockBytes = KU * kRowBytes;
    static constexpr int kWords = (kBlockBytes + 255) / 256;  // per lane
    static constexpr int kSlotElems = KU * N * R;
    static_assert(sizeof(IO) == 2, "bf16 operands");
    static_assert(kWords == 1 || kWords == 2 || kWords == 4, "C block of 4 .. 1024 bytes");
    __amdgpu_buffer_rsrc_t r;  // this walk's C rows, from its first row on
    SSM_LDS uint16_t *slot;    // the wave's kSlotElems elements
    uint32_t voff;             // the lane's first byte in a block (clamped into the block)
    __device__ __forceinline__ void init(const IO *C0, SSM_LDS uint16_t *s) {
        r = __builtin_amdgcn_make_buffer_rsrc(const_cast<IO *>(C0), 0, -1, kRsrcWord3);
        slot = s;
        voff = min((threadIdx.x & 63u) * 4u * kWords, (uint32_t)(kBlockBytes - 4 * kWords));
    }
    __device__ __forceinline__ void load(uint32_t (&w)[kWords], uint32_t row) const {
        const uint32_t so = row * (uint32_t)kRowBytes;
        if constexpr (kWords == 1) {
            w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, so, 0);
        } else if constexpr (kWords == 2) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, voff, so, 0);
            w[0] = t[0]; w[1] = t[1];
        } else {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, so, 0);
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = t[k];
        }
    }
    __device__ __forceinline__ void put(const uint32_t (&w)[kWords]) const {
        // with fewer than 64 * kWords words in a block the lanes past them only reread
        // the block's last words: they write nothing
        if constexpr (kBlockBytes < 256 * kWords)
            if ((threadIdx.x & 63u) * 4u * kWords >= (uint32_t)kBlockBytes) return;
        const uint32_t e0 = voff / 2u;  // the lane's first element
#pragma unroll
        for (int k = 0; k < kWords; ++k) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t e = e0 + (uint32_t)(2 * k + j);
                const uint32_t st = e / (uint32_t)(N * R), n = (e / R) % N, rr = e % R;
                slot[(st * R + rr) * N + n] = (uint16_t)(j ? w[k] >> 16 : w[k]);
            }
        }
    }
    // The lane's operands for step j of the block (rank 4g + l%4 at [4 g N + n]).
    __device__ __forceinline__ COpsLds<N> ops(int j) const {
        return COpsLds<N>{slot + (j * R + (int)(threadIdx.x & 3u)) * N};
    }
};

// Vector-memory instructions one block of KU steps issues: x, dt (and z) per step, the
// B staging loads on the matrix path and the C load when the outputs are on it too.
template <typename IO, int N, int R, bool GATED, int KU, bool WITH_C>
constexpr int block_vm_ops() {
    constexpr int vx = VecRaw<IO, R>::kBytes == 32 ? 2 : 1;
    return KU * (vx + 1 + (GATED ? vx : 0)) + (kMatInput<R> ? BStage<IO, N, R, KU>::kLoads : 0) +
           (WITH_C && kMatOutput<IO, N, R> ? 1 : 0);
}

// Calls body(i, x_i, dt_i, z_i, brow_i, cops_i) for i = 0 .. steps-1, with the next
// block of KU rows in flight while the current one is computed (as stream_steps does for
// scalar rows). brow_i is step i's row of B (an LDS pointer from the staging ring, or,
// in the ragged tail, a global pointer) on the matrix path, and unused (null) otherwise;
// cops_i gives the step's C operands of the matrix outputs (WITH_C with kMatOutput;
// CNone otherwise). B0, C0: the walk's first B and C rows (global); ring: the wave's 2
// B slots; cslot: the wave's C slot (WITH_C with kMatOutput only).
template <typename IO, int N, int R, bool GATED, int KU, bool WITH_C, typename Body>
__device__ __forceinline__ void mimo_steps(const VecStream<IO, R> &x, const RowStream<IO> &dt,
                                           const VecStream<IO, R> &z, const MimoStreams &o,
                                           const IO *B0, SSM_LDS char *ring, const IO *C0,
                                           SSM_LDS uint16_t *cslot, uint32_t steps, uint32_t prio_scale,
                                           Body &&body) {
    constexpr bool kMat = kMatInput<R>;
    constexpr bool kC = WITH_C && kMatOutput<IO, N, R>;
    constexpr int kOps = block_vm_ops<IO, N, R, GATED, KU, WITH_C>();
    typedef BStage<IO, N, R, KU> Stg;
    typedef CStage<uint16_t, N, R, KU> CStg;
    Stg st;
    CStg cst;
    if constexpr (kMat) {
        st.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<IO *>(B0), 0, -1, kRsrcWord3);
        st.ring = ring;
    }
    if constexpr (kC) cst.init((const uint16_t *)C0, cslot);
    // This block's staged rows are complete once only the next block's loads are pending.
    // On the matrix path a next block is always issued (the last block loads its own rows
    // again, into the idle buffer and slot), so that this wait is one straight-line
    // vmcnt(kOps): behind a branch the compiler's own wait tracking does not see it and
    // falls back to vmcnt(0) before each step's first use of x, which also waits for the
    // next block's loads.
    auto ready = [&]() {
        if constexpr (kMat) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(wait_vm(kOps));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto brow = [&](int slot, int j) {
        if constexpr (kMat) return st.row_at(slot, j);
        else return (const SSM_LDS char *)nullptr;
    };
    auto cops = [&](int j) {
        if constexpr (kC) return cst.ops(j);
        else return CNone{};
    };
    constexpr int CW = kC ? CStg::kWords : 1;
    auto load_block = [&](MimoBlock<IO, R, KU, CW> &buf, uint32_t row) {
        load_mimo_block<IO, R, GATED, KU>(buf, x, dt, z, o, row);
        if constexpr (kC) cst.load(buf.cw, row);
    };
    const uint32_t full = steps / KU;
    uint32_t i = 0;
    MimoBlock<IO, R, KU, CW> bufA, bufB;
    if (full > 0) {
        if constexpr (kMat) st.stage(0, 0);
        load_block(bufA, 0);
    }
    for (uint32_t k = 0; k < full; k += 2) {
        if (prio_scale) set_priority(steps - i, prio_scale);
        const bool more1 = k + 1 < full;
        if (kMat || more1) {
            const uint32_t nxt = more1 ? i + KU : i;
            if constexpr (kMat) st.stage(1, nxt);
            load_block(bufB, nxt);
        }
        ready();
        if constexpr (kC) cst.put(bufA.cw);
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, bufA.x[j], RowStream<IO>::widen(bufA.dt[j]), bufA.z[j], brow(0, j), cops(j));
        }
        i += KU;
        if (!more1) break;
        const bool more2 = k + 2 < full;
        if (kMat || more2) {
            const uint32_t nxt = more2 ? i + KU : i;
            if constexpr (kMat) st.stage(0, nxt);
            load_block(bufA, nxt);
        }
        ready();
        if constexpr (kC) cst.put(bufB.cw);
#pragma unroll
        for (int j = 0; j < KU; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            body(i + j, bufB.x[j], RowStream<IO>::widen(bufB.dt[j]), bufB.z[j], brow(1, j), cops(j));
        }
        i += KU;
    }
    if (prio_scale) __builtin_amdgcn_s_setprio(0);
    for (; i < steps; ++i) {  // ragged tail, one step at a time, B and C rows read directly
        const VecRaw<IO, R> xv = x.ld(o.vx, i * o.rbx);
        const float dv = dt.ld(o.vd, i * o.rbd);
        VecRaw<IO, R> zv{};
        if (GATED) zv = z.ld(o.vx, i * o.rbx);
        const char *g = kMat ? (const char *)B0 + (size_t)i * BStage<IO, N, R, KU>::kRowBytes : nullptr;
        if constexpr (kC) body(i, xv, dv, zv, g, COpsGlb<N, R>{(const uint16_t *)C0 + (size_t)i * N * R});
        else body(i, xv, dv, zv, g, CNone{});
    }
}

// A lane's batch row and channel. Lanes past the last channel keep running on the
// last channel (the matrix operations read operands from every lane of the wave) and
// store nothing.
struct LaneId {
    int64_t b, d;
    bool live;
};

__device__ __forceinline__ LaneId lane_id(const ScanArgs &a) {
    LaneId r;
    r.b = (int64_t)blockIdx.x / a.dblocks;
    const int64_t d = ((int64_t)blockIdx.x % a.dblocks) * a.threads + threadIdx.x;
    r.live = d < a.Dn;
    r.d = r.live ? d : a.Dn - 1;
    return r;
}

// The wave's staging ring for B rows (matrix path), in a block's LDS of 4 waves.
template <typename IO, int N, int R, int KU>
struct Ring {
    static constexpr int kBytes = kMatInput<R> ? 2 * BStage<IO, N, R, KU>::kSlotBytes : 16;
};

__device__ __forceinline__ MimoStreams mimo_offsets(const ScanArgs &a, int64_t d, int R, int eb) {
    MimoStreams o;
    o.vx = (uint32_t)d * (uint32_t)(R * eb);
    o.vd = (uint32_t)d * (uint32_t)eb;
    o.rbx = (uint32_t)(a.Dn * R * eb);
    o.rbd = (uint32_t)(a.Dn * eb);
    return o;
}

// Steps of x / z / y rows are R elements per channel: blocks of 4 steps for R <= 2,
// 2 for wider ranks with bf16 inputs and 1 with fp32 ones (keeps the ping-pong buffers
// within the register budget of the waves the rescan is compiled for).
template <typename IO, int R> constexpr int kMimoKU = R <= 2 ? 4 : sizeof(IO) == 4 ? 1 : 2;

// ---------------------------------------------------------------- chunk summary
template <typename IO, int N, int R>
__global__ __launch_bounds__(256) void k_mimo_summary(ScanArgs a) {
    constexpr int KU = kMimoKU<IO, R>;
    __shared__ __attribute__((aligned(16))) char ring_mem[4 * Ring<IO, N, R, KU>::kBytes];
    const LaneId ln = lane_id(a);
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t T = (uint32_t)a.T;  // every chunk that has a summary is full length
    constexpr int eb = (int)sizeof(IO);
    const MimoStreams o = mimo_offsets(a, ln.d, R, eb);
    float A2[N], h[N];
    float amax = -INFINITY;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        amax = fmaxf(amax, A2[n]);
        h[n] = 0.0f;
    }
    const int64_t t_row0 = ln.b * a.L + t0;  // row of (b, t0)
    const RowStream<IO> dts((const IO *)a.dt + t_row0 * a.Dn);
    const uint32_t ts = horizon_start<IO>(dts, o.vd, o.rbd, T, amax);
    const int64_t rw = t_row0 + ts;
    const VecStream<IO, R> xs((const IO *)a.x + rw * a.Dn * R);
    const RowStream<IO> dws((const IO *)a.dt + rw * a.Dn);
    const UniRow<IO, N * R> Bp(a.B, ln.b * a.L * N * R);
    SSM_LDS char *ring = (SSM_LDS char *)ring_mem + (threadIdx.x / 64) * Ring<IO, N, R, KU>::kBytes;
    double S = 0.0;  // sum of dt, needed only when the window is the whole chunk
    mimo_steps<IO, N, R, false, KU, false>(xs, dws, xs, o, (const IO *)a.B + rw * N * R, ring, nullptr,
                                           nullptr, T - ts, kSummaryPrioScale,
                                           [&](uint32_t i, const VecRaw<IO, R> &xr, float dv, const VecRaw<IO, R> &,
                                               auto brow, auto) {
        const int64_t t = t0 + ts + i;
        S += (double)dv;
        if constexpr (kMatInput<R>) {
            float v[N];
            mimo_bx<IO, N, R>(brow, xr, v);
#pragma unroll
            for (int n = 0; n < N; ++n) h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], dv * v[n]);
        } else {
            float xd[R];
#pragma unroll
            for (int r = 0; r < R; ++r) xd[r] = dv * xr.at(r);
#pragma unroll
            for (int n = 0; n < N; ++n)
                h[n] = __builtin_fmaf(e2(dv * A2[n]), h[n], mimo_input<R>(Bp, (t * N + n) * R, xd));
        }
    });
    if (!ln.live) return;
    const float Sf = (float)S;
    const size_t so = (((size_t)c * a.batch + ln.b) * a.Dn + ln.d) * N;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        a.sumP[so + n] = ts == 0 ? e2(A2[n] * Sf) : 0.0f;
        a.sumH[so + n] = h[n];
    }
}

// ---------------------------------------------------------------- rescan + epilogue
// Waves per SIMD the rescan is compiled for: 5 up to rank 4, 4 at rank 8 (the planner
// cuts the sequence into enough chunks for that many waves on every SIMD).
template <int R> constexpr int kMimoWavesPerSimd = R <= 4 ? 5 : 4;

template <typename IO, int N, int R, bool GATED>
__global__ __launch_bounds__(256, kMimoWavesPerSimd<R>) void k_mimo_scan(ScanArgs a) {
    constexpr int KU = kMimoKU<IO, R>;
    constexpr int kCSlot = kMatOutput<IO, N, R> ? CStage<uint16_t, N, R, KU>::kSlotElems : 8;
    __shared__ __attribute__((aligned(16))) char ring_mem[4 * Ring<IO, N, R, KU>::kBytes];
    __shared__ __attribute__((aligned(16))) uint16_t cslot_mem[4 * kCSlot];
    const LaneId ln = lane_id(a);
    const int c = blockIdx.y;
    const int64_t t0 = (int64_t)c * a.T;
    const uint32_t steps = (uint32_t)(min(a.L, t0 + a.T) - t0);
    const size_t col = (size_t)(ln.b * a.Dn + ln.d) * N;
    const float *hin = c == 0 ? (a.h0 ? a.h0 + col : nullptr)
                              : a.sumH + (size_t)(c - 1) * a.batch * a.Dn * N + col;
    constexpr int eb = (int)sizeof(IO);
    const MimoStreams o = mimo_offsets(a, ln.d, R, eb);
    float A2[N], h[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        A2[n] = a.A[ln.d * N + n] * kLog2e;
        h[n] = hin ? hin[n] : 0.0f;
    }
    const float Dd = a.D[ln.d];
    const int64_t t_row0 = ln.b * a.L + t0;
    const VecStream<IO, R> xs((const IO *)a.x + t_row0 * a.Dn * R),
        zs(GATED ? (const IO *)a.z + t_row0 * a.Dn * R : (const IO *)a.x + t_row0 * a.Dn * R),
        ys((IO *)a.y + t_row0 * a.Dn * R);
    const RowStream<IO> dts((const IO *)a.dt + t_row0 * a.Dn);
    const UniRow<IO, N * R> Bp(a.B, ln.b * a.L * N * R);
    const UniRow<IO, N * R> Cp(a.C, ln.b * a.L * N * R);
    SSM_LDS char *ring = (SSM_LDS char *)ring_mem + (threadIdx.x / 64) * Ring<IO, N, R, KU>::kBytes;
    SSM_LDS uint16_t *cslot = (SSM_LDS uint16_t *)cslot_mem + (threadIdx.x / 64) * kCSlot;
    mimo_steps<IO, N, R, GATED, KU, true>(xs, dts, zs, o, (const IO *)a.B + t_row0 * N * R, ring,
                                          (const IO *)a.C + t_row0 * N * R, cslot, steps, steps,
                                          [&](uint32_t i, const VecRaw<IO, R> &xr, float dv, const VecRaw<IO, R> &zr,
                                              auto brow, auto cops) {
        const int64_t t = t0 + i;
        float xv[R], acc[R], yv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) xv[r] = xr.at(r);
        mimo_update<IO, N, R, kMatInput<R>>(h, A2, dv, xr, xv, Bp, Cp, brow, cops, t * N * R, acc);
        mimo_out<IO, R, GATED>(Dd, xv, acc, zr, yv);
        if (ln.live) ys.st(o.vx, i * o.rbx, yv);
    });
    if (!ln.live) return;
    if (c == a.n_chunks - 1 && a.h_final) {
#pragma unroll
        for (int n = 0; n < N; ++n) a.h_final[col + n] = h[n];
    }
}

// ---------------------------------------------------------------- decode step
// One token for every (layer, sequence, channel). One lane per channel holds the
// channel's N states; B_t and C_t are one row per (layer, sequence), the same for the
// whole block (grid y = sequence, z = layer), so they come in through the scalar unit.
// A block's 256 channels own one contiguous run of state: it is moved between HBM and
// LDS with coalesced, streaming 16-byte accesses (it is read and written once per
// token), and each lane reads and writes its channel's row of LDS. Rows are padded to
// P floats so that the 16 lanes of one LDS access start on distinct banks. A is read
// per lane from its own rows: it is the same for every sequence of a layer, so those
// reads are served by the caches (staging it through LDS as well halved the blocks
// per CU and made the call slower: 71.7 against 57.7 us on the 28 x 256 x 8192 decode).
typedef float f4v __attribute__((ext_vector_type(4)));

template <int N> constexpr int kLdsRow = N == 16 ? 20 : N == 8 ? 12 : N;

// dst[c * P + n] = src[c * N + n] for the block's nch channels (thread tid of 256),
// streaming loads.
template <int N>
__device__ __forceinline__ void rows_to_lds(float *dst, const float *src, int nch, int tid) {
    constexpr int P = kLdsRow<N>;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            const int v = tid + 256 * j;  // float4 index in the block's run
            if (v < nch * (N / 4)) {
                const f4v q = __builtin_nontemporal_load((const f4v *)src + v);
                const int c = (4 * v) / N, n = (4 * v) % N;
                *(f4v *)(dst + c * P + n) = q;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int e = tid + 256 * j;
            if (e < nch * N) dst[(e / N) * P + e % N] = src[e];
        }
    }
}

// dst[c * N + n] = src[c * P + n], streaming stores.
template <int N>
__device__ __forceinline__ void lds_to_rows(float *dst, const float *src, int nch, int tid) {
    constexpr int P = kLdsRow<N>;
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int j = 0; j < N / 4; ++j) {
            const int v = tid + 256 * j;
            if (v < nch * (N / 4)) {
                const int c = (4 * v) / N, n = (4 * v) % N;
                __builtin_nontemporal_store(*(const f4v *)(src + c * P + n), (f4v *)dst + v);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int e = tid + 256 * j;
            if (e < nch * N) dst[e] = src[(e / N) * P + e % N];
        }
    }
}

template <typename IO, int N, int R, bool GATED>
__global__ __launch_bounds__(256) void k_mimo_step(StepArgs a) {
    constexpr int P = kLdsRow<N>;
    __shared__ __attribute__((aligned(16))) float sh[256 * P];  // the block's states

    const int tid = (int)threadIdx.x;
    const int64_t d0 = (int64_t)blockIdx.x * 256;
    const int nch = (int)min((int64_t)256, a.Dn - d0);  // channels of this block
    const int64_t l = blockIdx.z;
    const int64_t lq = l * a.n_seq + blockIdx.y;
    const bool live = tid < nch;
    const int64_t d = d0 + (live ? tid : nch - 1);
    const int64_t ch = lq * a.Dn + d;
    // the lane's own token inputs first, then the block's state and A through LDS
    const VecRaw<IO, R> xr = ld_vec<IO, R>((const IO *)a.x + ch * R);
    VecRaw<IO, R> zr{};
    if (GATED) zr = ld_vec<IO, R>((const IO *)a.z + ch * R);
    const float dv = Io<IO>::ld((const IO *)a.dt + ch);
    const float Dd = a.D[l * a.Dn + d];
    float *hblk = a.h + (lq * a.Dn + d0) * N;
    rows_to_lds<N>(sh, hblk, nch, tid);

    float h[N], A2[N];
    const float *Ap = a.A + (l * a.Dn + d) * N;  // shared by every sequence: cached
#pragma unroll
    for (int n = 0; n < N; ++n) A2[n] = Ap[n] * kLog2e;
    __syncthreads();
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = sh[tid * P + n];
    const UniRow<IO, N * R> Bp(a.B, lq * N * R), Cp(a.C, lq * N * R);
    float xv[R], acc[R], yv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xv[r] = xr.at(r);
    mimo_update<IO, N, R, false>(h, A2, dv, xr, xv, Bp, Cp, (const char *)nullptr, CNone{}, 0, acc);
    mimo_out<IO, R, GATED>(Dd, xv, acc, zr, yv);
#pragma unroll
    for (int n = 0; n < N; ++n) sh[tid * P + n] = h[n];
    if (live) st_vec<IO, R>((IO *)a.y + ch * R, yv);
    __syncthreads();
    lds_to_rows<N>(hblk, sh, nch, tid);
}

template <typename IO, int N, int R>
hipError_t launch_step_t(const StepArgs &a, bool gated, hipStream_t s) {
    const dim3 grid((unsigned)((a.Dn + 255) / 256), (unsigned)a.n_seq, (unsigned)a.n_layers);
    if (gated) hipLaunchKernelGGL((k_mimo_step<IO, N, R, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_mimo_step<IO, N, R, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename IO, int R>
hipError_t launch_step_n(const StepArgs &a, int d_state, bool gated, hipStream_t s) {
    switch (d_state) {
        case 1: return launch_step_t<IO, 1, R>(a, gated, s);
        case 2: return launch_step_t<IO, 2, R>(a, gated, s);
        case 4: return launch_step_t<IO, 4, R>(a, gated, s);
        case 8: return launch_step_t<IO, 8, R>(a, gated, s);
        case 16: return launch_step_t<IO, 16, R>(a, gated, s);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_step_io(const StepArgs &a, int d_state, bool gated, hipStream_t s) {
    switch (a.rank) {
        case 1: return launch_step_n<IO, 1>(a, d_state, gated, s);
        case 2: return launch_step_n<IO, 2>(a, d_state, gated, s);
        case 4: return launch_step_n<IO, 4>(a, d_state, gated, s);
        case 8: return launch_step_n<IO, 8>(a, d_state, gated, s);
    }
    return hipErrorInvalidValue;
}

inline void mark(hipEvent_t const *ev, int i, hipStream_t s) {
    if (ev) (void)hipEventRecord(ev[i], s);
}

template <typename IO, int N, int R>
hipError_t launch_t(const ScanArgs &a, bool gated, hipStream_t s, hipEvent_t const *ev) {
    const dim3 blk(a.threads);
    const unsigned gx = (unsigned)(a.batch * a.dblocks);
    mark(ev, 0, s);
    if (a.n_chunks > 1)
        hipLaunchKernelGGL((k_mimo_summary<IO, N, R>), dim3(gx, a.n_chunks - 1), blk, 0, s, a);
    mark(ev, 1, s);
    hipError_t e = launch_carry(a, N, s);
    if (e != hipSuccess) return e;
    mark(ev, 2, s);
    if (gated)
        hipLaunchKernelGGL((k_mimo_scan<IO, N, R, true>), dim3(gx, a.n_chunks), blk, 0, s, a);
    else
        hipLaunchKernelGGL((k_mimo_scan<IO, N, R, false>), dim3(gx, a.n_chunks), blk, 0, s, a);
    mark(ev, 3, s);
    return hipGetLastError();
}

template <typename IO, int R>
hipError_t launch_n(const ScanArgs &a, int d_state, bool gated, hipStream_t s, hipEvent_t const *ev) {
    switch (d_state) {
        case 1: return launch_t<IO, 1, R>(a, gated, s, ev);
        case 2: return launch_t<IO, 2, R>(a, gated, s, ev);
        case 4: return launch_t<IO, 4, R>(a, gated, s, ev);
        case 8: return launch_t<IO, 8, R>(a, gated, s, ev);
        case 16: return launch_t<IO, 16, R>(a, gated, s, ev);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
hipError_t launch_io(const ScanArgs &a, int d_state, bool gated, hipStream_t s, hipEvent_t const *ev) {
    switch (a.rank) {
        case 1: return launch_n<IO, 1>(a, d_state, gated, s, ev);
        case 2: return launch_n<IO, 2>(a, d_state, gated, s, ev);
        case 4: return launch_n<IO, 4>(a, d_state, gated, s, ev);
        case 8: return launch_n<IO, 8>(a, d_state, gated, s, ev);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_mimo(const ScanArgs &a, int io, int d_state, bool gated, hipStream_t s,
                            hipEvent_t const *ev) {
    return io == 0 ? launch_io<float>(a, d_state, gated, s, ev)
                   : launch_io<bf16_bits>(a, d_state, gated, s, ev);
}

hipError_t launch_step_mimo(const StepArgs &a, int io, int d_state, bool gated, hipStream_t s) {
    return io == 0 ? launch_step_io<float>(a, d_state, gated, s)
                   : launch_step_io<bf16_bits>(a, d_state, gated, s);
}

}  // namespace ssm
