// api.cpp -- the C ABI of libssmscan: argument checks, chunk planning, dispatch.
//
// Every check runs on the host before anything is enqueued, so a rejected call
// leaves all outputs untouched. Kernels are enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "ssm_internal.h"
#include "ssm_scan.h"

namespace {

thread_local char g_err[512] = "";

ssm_status fail(ssm_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

ssm_status ok() {
    g_err[0] = '\0';
    return SSM_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_state(int32_t n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

bool valid_rank(int32_t r) { return r == 1 || r == 2 || r == 4 || r == 8; }

size_t io_bytes(ssm_dtype io) { return io == SSM_BF16 ? 2 : 4; }

// Waves wanted per launch for the chunk rescan: as many as the rescan kernel is
// compiled to keep resident per SIMD, on every SIMD of the device. One wave more than a
// round holds would start a second, mostly idle round, so the count must not exceed it.
//
// Device properties cache: the compute-unit count of each device, queried once (the
// first plan made while that device is current) and kept for the process. A CDNA
// compute unit has four SIMDs. SSMSCAN_CU_COUNT (a positive integer in the environment
// when the device is first queried) replaces the queried count, to plan for another
// part or partition. With no device to query (no GPU, or the HIP runtime reports an
// error) the plan assumes MI355X's 256 compute units and caches nothing.
constexpr int64_t kSimdsPerCu = 4;
constexpr int32_t kDefaultCus = 256;
constexpr int kMaxDevices = 64;
std::mutex g_prop_mu;
int32_t g_cus[kMaxDevices];  // 0: not queried yet

int32_t env_cus() {
    const char *e = getenv("SSMSCAN_CU_COUNT");
    const long v = e ? strtol(e, nullptr, 10) : 0;
    return v > 0 && v < (1 << 20) ? (int32_t)v : 0;
}

int64_t device_simds() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();  // leave no error behind for the next launch check
        const int32_t e = env_cus();
        return (int64_t)(e ? e : kDefaultCus) * kSimdsPerCu;
    }
    std::lock_guard<std::mutex> lock(g_prop_mu);
    if (!g_cus[dev]) {
        int32_t cus = env_cus();
        if (!cus) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
                cus = v;
            else
                (void)hipGetLastError();
        }
        if (!cus) return (int64_t)kDefaultCus * kSimdsPerCu;  // not cached: try again next time
        g_cus[dev] = cus;
    }
    return (int64_t)g_cus[dev] * kSimdsPerCu;
}

// Waves per SIMD each rescan is compiled for (its __launch_bounds__ minimum, or what
// its registers allow).
enum class Family { Plain, Fused, Complex, Mimo, Backward, TrapWeighted };
int32_t waves_per_simd(Family f, int32_t rank = 1) {
    switch (f) {
        case Family::Plain: return 5;     // plain and exponential-trapezoidal rescans
        case Family::TrapWeighted: return 5;  // its rescan prefetches 2 rows at a time
        case Family::Complex: return 5;
        case Family::Mimo: return rank <= 4 ? 5 : 4;
        default: return 4;                // input stage, backward
    }
}
// Lanes per channel: the complex-state kernels spread a channel's states over 4 lanes
// (fewer states: one lane each); the others keep a channel in one lane.
int64_t lanes_per_channel(bool cplx, int32_t d_state) {
    return cplx ? std::min<int32_t>(d_state, 4) : 1;
}
constexpr int64_t kMinChunk = 64;       // shortest chunk the planner picks
constexpr int64_t kMaxChunks = 65535;   // grid y limit
constexpr size_t kWsAlign = 256;

int64_t auto_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int64_t target_waves) {
    if (L <= 0) return 1;
    const int64_t waves_per_chunk = std::max<int64_t>(1, batch * ((d_inner + 63) / 64));
    int64_t chunks = (target_waves + waves_per_chunk - 1) / waves_per_chunk;
    chunks = std::min(chunks, (L + kMinChunk - 1) / kMinChunk);
    chunks = std::max<int64_t>(chunks, 1);
    return (L + chunks - 1) / chunks;
}

struct Plan {
    int64_t T;
    int32_t n_chunks;
    size_t ws_bytes;
};

// waves_per_simd: what the rescan of the entry point is compiled for (5 for the plain,
// trapezoidal, complex and MIMO rescans up to rank 4; 4 for the input stage, MIMO rank 8
// and the backward's own plan).
// multiple: with several chunks, chunk lengths are rounded down to a multiple of it (the
// training forward's chunks start where a stored state belongs).
ssm_status make_plan(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state, int64_t chunk_len,
                     bool cplx, Plan *p, int32_t rank = 1, int32_t waves_per_simd = 4,
                     int64_t multiple = 1) {
    if (batch < 0 || L < 0 || d_inner < 1) return fail(SSM_ERR_SHAPE, "batch/L must be >= 0 and d_inner >= 1");
    if (!valid_state(d_state)) return fail(SSM_ERR_UNSUPPORTED, "d_state %d not in {1,2,4,8,16}", d_state);
    if (chunk_len < 0) return fail(SSM_ERR_UNSUPPORTED, "chunk_len must be >= 0");
    // keep every element index inside int64 with margin
    const double elems = (double)batch * (double)L * (double)d_inner;
    if (elems > 4.0e18 || (double)batch * d_inner > 2.0e9)
        return fail(SSM_ERR_SHAPE, "problem too large");
    // A chunk spans less than 2 GiB of every [rows][d_inner] stream (4-byte elements
    // at most), so the kernels address a chunk with 32-bit byte offsets.
    // (MIMO rows of x, z and y hold rank elements per channel.)
    const int64_t cap = std::max<int64_t>(1, ((int64_t)1 << 31) / (d_inner * rank * 4) - 1);
    int64_t T = chunk_len > 0 ? std::min(chunk_len, std::max<int64_t>(L, 1))
                              : auto_chunk_len(batch, L, d_inner * lanes_per_channel(cplx, d_state),
                                               waves_per_simd * device_simds());
    T = std::min(T, cap);
    // MIMO: a chunk's rows of B (d_state * rank elements each) also span less than 2 GiB,
    // since the matrix path stages them through buffer loads with 32-bit offsets.
    if (rank > 1) T = std::min(T, std::max<int64_t>(1, ((int64_t)1 << 31) / ((int64_t)d_state * rank * 4) - 1));
    if (multiple > 1 && T < L) T = std::max(multiple, T / multiple * multiple);
    const int64_t n_chunks = L > 0 ? (L + T - 1) / T : 1;
    if (n_chunks > kMaxChunks) return fail(SSM_ERR_UNSUPPORTED, "chunk_len gives %lld chunks (max %lld)", (long long)n_chunks, (long long)kMaxChunks);
    p->T = T;
    p->n_chunks = (int32_t)n_chunks;
    const size_t per = (size_t)batch * d_inner * d_state * sizeof(float) * (cplx ? 2 : 1);
    const size_t one = ((per * (size_t)(n_chunks - 1)) + kWsAlign - 1) / kWsAlign * kWsAlign;
    p->ws_bytes = n_chunks > 1 ? 2 * one : 0;
    return ok();
}

ssm_status launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The MambaBlock input stage of the fused entry points.
struct InputStage {
    const float *conv_w, *conv_b, *dt_bias;
    int32_t conv_k;
    const void *conv_state0;  // prefill only
    void *conv_state;         // prefill: conv_state_out; decode: the state, in place
    void *u_out = nullptr, *dt_out = nullptr;  // the fused training forward: u and dt out
};

// The exponential-trapezoidal entry points: the input before the first step (prefill:
// [batch][Dn] and [batch][N]; decode: the previous token's x and B; both or neither),
// and the weight of each step's current input (laid out like dt; null: 1/2).
struct Trap {
    const void *x_prev, *B_prev, *lam;
};

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

ssm_status check_input_stage(const InputStage &in, size_t eb) {
    if (in.conv_k < 0 || in.conv_k > 4) return fail(SSM_ERR_UNSUPPORTED, "conv_k %d not in 0..4", in.conv_k);
    if (in.conv_k > 0 && !in.conv_w) return fail(SSM_ERR_NULL, "conv_w is required when conv_k > 0");
    if (!aligned(in.conv_w, 4) || !aligned(in.conv_b, 4) || !aligned(in.dt_bias, 4) ||
        !aligned(in.conv_state0, eb) || !aligned(in.conv_state, eb))
        return fail(SSM_ERR_ALIGN, "pointer alignment (conv_w, conv_b, dt_bias 4 B; conv state element)");
    return ok();
}

ssm_status scan_common(const void *x, const void *dt, const float *A, const void *B, const void *C,
                       const float *D, const void *z, const float *h0, void *y, float *h_final,
                       int64_t batch, int64_t L, int64_t d_inner, int32_t d_state, ssm_dtype io,
                       int64_t chunk_len, void *workspace, size_t workspace_bytes,
                       void *hip_stream, bool cplx, void *const *events = nullptr,
                       int32_t n_events = 0, const InputStage *in = nullptr,
                       const Trap *trap = nullptr, int32_t rank = 0, bool use_scratch = false,
                       float *states = nullptr) {
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_DTYPE, "io dtype %d unknown", (int)io);
    const bool mimo = rank != 0;
    if (mimo && !valid_rank(rank)) return fail(SSM_ERR_UNSUPPORTED, "rank %d not in {1,2,4,8}", rank);
    Plan plan;
    const Family fam = cplx ? Family::Complex : in ? Family::Fused : mimo ? Family::Mimo
                     : (trap && trap->lam) ? Family::TrapWeighted : Family::Plain;
    ssm_status st = make_plan(batch, L, d_inner, d_state, chunk_len, cplx, &plan, mimo ? rank : 1,
                              waves_per_simd(fam, rank), states ? ssm::kStateEvery : 1);
    if (st != SSM_OK) return st;
    const bool work = batch > 0 && L > 0;
    if (work && (!x || !dt || !A || !B || !C || !D || !y))
        return fail(SSM_ERR_NULL, "x, dt, A, B, C, D and y are required");
    if (states) {
        if (!aligned(states, 16)) return fail(SSM_ERR_ALIGN, "states must be 16-byte aligned");
        if ((double)batch * d_inner * d_state * 4.0 >= 2147483648.0)
            return fail(SSM_ERR_UNSUPPORTED, "stored states need batch * d_inner * d_state * 4 below 2 GiB");
    }
    const size_t eb = io_bytes(io);
    if (!aligned(x, eb) || !aligned(dt, eb) || !aligned(z, eb) || !aligned(y, eb) ||
        !aligned(B, 4) || !aligned(C, 4) || !aligned(A, 16) || !aligned(D, 4) ||
        !aligned(h0, 16) || !aligned(h_final, 16))
        return fail(SSM_ERR_ALIGN, "pointer alignment (A, h0, h_final 16 B; B, C, D 4 B; x, dt, z, y element)");
    if (mimo) {
        // x, z and y are read and written R elements (up to 16 bytes) at a time.
        const size_t va = std::min<size_t>(16, (size_t)rank * eb);
        if (!aligned(x, va) || !aligned(z, va) || !aligned(y, va) ||
            (rank >= 4 && (!aligned(B, va) || !aligned(C, va))))
            return fail(SSM_ERR_ALIGN, "pointer alignment (x, z, y, and B, C for rank >= 4: min(16, rank * element) bytes)");
        if ((double)batch * L * d_inner * rank > 4.0e18)
            return fail(SSM_ERR_SHAPE, "problem too large");
    }
    if (events && n_events != 4) return fail(SSM_ERR_NULL, "profiling needs exactly 4 events");
    if (events)
        for (int i = 0; i < 4; ++i)
            if (!events[i]) return fail(SSM_ERR_NULL, "profiling event %d is NULL", i);
    // conv state rows carried between calls: conv_k - 1 per batch row
    const int64_t conv_rows = in && in->conv_k > 1 ? in->conv_k - 1 : 0;
    if (in) {
        st = check_input_stage(*in, eb);
        if (st != SSM_OK) return st;
        const size_t stream_bytes = (size_t)(batch * L * d_inner) * eb;
        const size_t state_bytes = (size_t)(batch * conv_rows * d_inner) * eb;
        // The rescan of chunk c reads the last conv_k-1 inputs of chunk c-1 while that
        // chunk's y and the final conv state are written.
        if (in->conv_k > 1 && overlaps(y, stream_bytes, x, stream_bytes))
            return fail(SSM_ERR_UNSUPPORTED, "y must not overlap x_in when the convolution is fused");
        if (overlaps(in->conv_state, state_bytes, x, stream_bytes) ||
            overlaps(in->conv_state, state_bytes, in->conv_state0, state_bytes))
            return fail(SSM_ERR_UNSUPPORTED, "conv_state_out must not overlap x_in or conv_state0");
    }
    if (trap) {
        if ((trap->x_prev == nullptr) != (trap->B_prev == nullptr))
            return fail(SSM_ERR_NULL, "x_prev and B_prev are given together or not at all");
        if (!aligned(trap->x_prev, eb) || !aligned(trap->B_prev, 4) || !aligned(trap->lam, eb))
            return fail(SSM_ERR_ALIGN, "pointer alignment (x_prev, lam element, B_prev 4 B)");
        // The rescan of chunk c reads the last row of chunk c-1 while y is written.
        const size_t stream_bytes = (size_t)(batch * L * d_inner) * eb;
        if (overlaps(y, stream_bytes, x, stream_bytes) ||
            overlaps(y, stream_bytes, trap->x_prev, (size_t)(batch * d_inner) * eb) ||
            overlaps(y, stream_bytes, trap->lam, stream_bytes))
            return fail(SSM_ERR_UNSUPPORTED, "y must not overlap x, x_prev or lam in the trapezoidal scan");
    }
    hipStream_t s = (hipStream_t)hip_stream;
    const int64_t state_floats = batch * d_inner * d_state * (cplx ? 2 : 1);
    if (!work) {
        if (h_final) {
            st = launch_status(ssm::launch_state_fill(h_final, h0, state_floats, s), "state fill");
            if (st != SSM_OK) return st;
        }
        if (conv_rows && in->conv_state)
            return launch_status(ssm::launch_elem_fill(in->conv_state, in->conv_state0,
                                                       batch * conv_rows * d_inner, (int)eb, s),
                                 "conv state fill");
        return ok();
    }
    if (use_scratch && plan.ws_bytes > 0) {
        // the no-allocation entry point: the device's own scratch array is the workspace
        if (plan.ws_bytes > (size_t)SSM_NOALLOC_SCRATCH_BYTES)
            return fail(SSM_ERR_WORKSPACE,
                        "this chunk plan needs %zu bytes of scratch; ssm_scan_fwd_noalloc has %zu "
                        "(use a longer chunk_len, or ssm_scan_fwd_ex with a workspace)",
                        plan.ws_bytes, (size_t)SSM_NOALLOC_SCRATCH_BYTES);
        st = launch_status(ssm::scratch_buffer(&workspace, &workspace_bytes), "scratch lookup");
        if (st != SSM_OK) return st;
    }
    if (plan.ws_bytes > 0) {
        if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", plan.ws_bytes);
        if (workspace_bytes < plan.ws_bytes)
            return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, plan.ws_bytes);
        if (!aligned(workspace, kWsAlign)) return fail(SSM_ERR_ALIGN, "workspace must be 256-byte aligned");
    }
    ssm::ScanArgs a{};
    a.x = x; a.dt = dt; a.B = B; a.C = C; a.z = z;
    a.A = A; a.D = D; a.h0 = h0;
    a.y = y; a.h_final = h_final;
    a.sumP = (float *)workspace;
    a.sumH = plan.ws_bytes ? (float *)((char *)workspace + plan.ws_bytes / 2) : nullptr;
    a.batch = batch; a.L = L; a.Dn = d_inner;
    a.T = plan.T; a.n_chunks = plan.n_chunks;
    a.rank = mimo ? rank : 1;
    a.threads = (int32_t)std::min<int64_t>(256, (d_inner + 63) / 64 * 64);
    a.dblocks = (int32_t)((d_inner + a.threads - 1) / a.threads);
    const int iot = io == SSM_BF16 ? 1 : 0;
    hipEvent_t const *ev = (hipEvent_t const *)events;
    hipError_t e;
    if (in) {
        a.conv_k = in->conv_k;
        a.conv_w = in->conv_k > 0 ? in->conv_w : nullptr;
        a.conv_b = in->conv_k > 0 ? in->conv_b : nullptr;
        a.conv_state0 = conv_rows ? in->conv_state0 : nullptr;
        a.conv_state_out = conv_rows ? in->conv_state : nullptr;
        a.dt_bias = in->dt_bias;
        a.states = states;  // the fused training forward (with u_out, dt_out), or null
        a.u_out = in->u_out;
        a.dt_out = in->dt_out;
        e = ssm::launch_scan_fused(a, iot, d_state, z != nullptr, s, ev);
    } else if (trap) {
        a.x_prev = trap->x_prev;
        a.B_prev = trap->B_prev;
        a.lam = trap->lam;
        e = ssm::launch_scan_trap(a, iot, d_state, z != nullptr, s, ev);
    } else if (mimo) {
        e = ssm::launch_scan_mimo(a, iot, d_state, z != nullptr, s, ev);
    } else if (states) {
        a.states = states;
        e = ssm::launch_scan_save(a, iot, d_state, z != nullptr, s, ev);
    } else {
        e = cplx ? ssm::launch_scan_complex(a, iot, d_state, z != nullptr, s, ev)
                 : ssm::launch_scan_real(a, iot, d_state, z != nullptr, s, ev);
    }
    return launch_status(e, "scan launch");
}

ssm_status step_common(float *h, const void *x, const void *dt, const float *A, const void *B,
                       const void *C, const float *D, const void *z, void *y, int64_t n_layers,
                       int64_t n_seq, int64_t d_inner, int32_t d_state, ssm_dtype io,
                       void *hip_stream, bool cplx, bool replay,
                       const InputStage *in = nullptr, const Trap *trap = nullptr,
                       int32_t rank = 0) {
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_DTYPE, "io dtype %d unknown", (int)io);
    if (n_layers < 0 || n_seq < 0 || d_inner < 1) return fail(SSM_ERR_SHAPE, "n_layers/n_seq must be >= 0 and d_inner >= 1");
    if (!valid_state(d_state)) return fail(SSM_ERR_UNSUPPORTED, "d_state %d not in {1,2,4,8,16}", d_state);
    const bool mimo = rank != 0;
    if (mimo && !valid_rank(rank)) return fail(SSM_ERR_UNSUPPORTED, "rank %d not in {1,2,4,8}", rank);
    if ((double)n_layers * n_seq * d_inner * 16.0 > 4.0e18) return fail(SSM_ERR_SHAPE, "problem too large");
    if (n_layers > 65535 || n_seq > 65535 || d_inner > ((int64_t)1 << 28))
        return fail(SSM_ERR_SHAPE, "n_layers and n_seq must be <= 65535, d_inner <= 2^28");
    if (n_layers == 0 || n_seq == 0) return ok();
    if (!h || !x || !dt || !A || !B || !C || !D || !y)
        return fail(SSM_ERR_NULL, "h, x_t, dt_t, A, B_t, C_t, D and y_t are required");
    const size_t eb = io_bytes(io);
    // B_t and C_t rows are read K values at a time: K = 4 states per lane for
    // d_state >= 4 (real), else d_state; complex rows are read one value at a time.
    // MIMO rows of B_t and C_t go through the scalar unit (4-byte aligned); from rank 4 B_t
    // is also read as matrix operands, min(16, rank * element) bytes at a time.
    const size_t bc = mimo ? 4 : cplx ? eb : eb * (size_t)std::min<int32_t>(d_state, 4);
    if (mimo && rank >= 4 && !aligned(B, std::min<size_t>(16, (size_t)rank * eb)))
        return fail(SSM_ERR_ALIGN, "pointer alignment (B_t for rank >= 4: min(16, rank * element) bytes)");
    if (!aligned(h, 16) || !aligned(A, 16) || !aligned(x, eb) || !aligned(dt, eb) ||
        !aligned(z, eb) || !aligned(y, eb) || !aligned(B, bc) || !aligned(C, bc) || !aligned(D, 4))
        return fail(SSM_ERR_ALIGN, "pointer alignment (h, A 16 B; B_t, C_t min(d_state,4) elements; others element)");
    if (trap) {
        if ((trap->x_prev == nullptr) != (trap->B_prev == nullptr))
            return fail(SSM_ERR_NULL, "x_prev and B_prev are given together or not at all");
        if (!aligned(trap->x_prev, eb) || !aligned(trap->B_prev, bc) || !aligned(trap->lam, eb))
            return fail(SSM_ERR_ALIGN, "pointer alignment (x_prev, lam_t element; B_prev as B_t)");
    }
    if (mimo) {
        const size_t va = std::min<size_t>(16, (size_t)rank * eb);
        if (!aligned(x, va) || !aligned(z, va) || !aligned(y, va))
            return fail(SSM_ERR_ALIGN, "pointer alignment (x_t, z_t, y_t: min(16, rank * element) bytes)");
    }
    ssm::StepArgs a{};
    a.h = h; a.x = x; a.dt = dt; a.B = B; a.C = C; a.z = z; a.A = A; a.D = D; a.y = y;
    a.n_layers = n_layers; a.n_seq = n_seq; a.Dn = d_inner;
    const int iot = io == SSM_BF16 ? 1 : 0;
    hipStream_t s = (hipStream_t)hip_stream;
    hipError_t e;
    if (in) {
        ssm_status st = check_input_stage(*in, eb);
        if (st != SSM_OK) return st;
        if (in->conv_k > 1 && !in->conv_state)
            return fail(SSM_ERR_NULL, "conv_state is required when conv_k > 1");
        a.conv_k = in->conv_k;
        a.conv_w = in->conv_k > 0 ? in->conv_w : nullptr;
        a.conv_b = in->conv_k > 0 ? in->conv_b : nullptr;
        a.conv_state = in->conv_k > 1 ? in->conv_state : nullptr;
        a.dt_bias = in->dt_bias;
        e = ssm::launch_step_fused(a, iot, d_state, z != nullptr, replay, s);
    } else if (trap) {
        a.x_prev = trap->x_prev;
        a.B_prev = trap->B_prev;
        a.lam = trap->lam;
        e = ssm::launch_step_trap(a, iot, d_state, z != nullptr, replay, s);
    } else if (mimo) {
        a.rank = rank;
        e = ssm::launch_step_mimo(a, iot, d_state, z != nullptr, s);
    } else {
        e = cplx ? ssm::launch_step_complex(a, iot, d_state, z != nullptr, replay, s)
                 : ssm::launch_step_real(a, iot, d_state, z != nullptr, replay, s);
    }
    return launch_status(e, "step launch");
}

// Backward plan: the forward's chunks, with the length a multiple of kSub when there is
// more than one chunk, so that every chunk starts on a sub-chunk boundary.
struct BwdPlan {
    Plan fwd;
    size_t off[8];  // byte offsets of sumP, sumH, revQ, revG, ckpt, partA, partD, partBC
    size_t bytes;
    int32_t waves, threads, dblocks;
    int64_t ck_rows;  // stored-state rows per chunk
};

size_t ws_round(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// saved: the states come from the training forward (chunks start at multiples of
// kStateEvery, and the workspace holds no states of its own).
ssm_status make_bwd_plan(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                         int64_t chunk_len, BwdPlan *p, bool saved = false) {
    ssm_status st = make_plan(batch, L, d_inner, d_state, chunk_len, false, &p->fwd, 1,
                              waves_per_simd(Family::Backward));
    if (st != SSM_OK) return st;
    if (p->fwd.n_chunks > 1) {
        // (from stored states, chunk lengths are rounded as ssm_scan_fwd_save rounds them)
        const int64_t m = saved ? ssm::kStateEvery : ssm::kSub;
        int64_t T = saved ? std::max<int64_t>(m, p->fwd.T / m * m) : p->fwd.T / m * m;
        if (T < m) return fail(SSM_ERR_UNSUPPORTED, "chunk_len must be at least %d for the backward", (int)m);
        const int64_t n = (L + T - 1) / T;
        if (n > kMaxChunks) return fail(SSM_ERR_UNSUPPORTED, "chunk_len gives %lld chunks (max %lld)", (long long)n, (long long)kMaxChunks);
        p->fwd.T = T;
        p->fwd.n_chunks = (int32_t)n;
    }
    if ((double)batch * d_inner * d_state * 4.0 >= 2147483648.0)
        return fail(SSM_ERR_UNSUPPORTED, "the backward needs batch * d_inner * d_state * 4 below 2 GiB");
    p->threads = (int32_t)std::min<int64_t>(256, (d_inner + 63) / 64 * 64);
    p->dblocks = (int32_t)((d_inner + p->threads - 1) / p->threads);
    p->waves = p->dblocks * (p->threads / 64);
    const size_t M = (size_t)batch * d_inner * d_state * sizeof(float);
    const size_t C = (size_t)p->fwd.n_chunks;
    p->ck_rows = (std::min<int64_t>(p->fwd.T, L) + ssm::kStateEvery - 1) / ssm::kStateEvery;
    const size_t sizes[8] = {(C - 1) * M, (C - 1) * M, (C - 1) * M, (C - 1) * M,
                             saved ? 0 : C * (size_t)p->ck_rows * M, C * M,
                             C * (size_t)batch * d_inner * sizeof(float),
                             (size_t)batch * L * p->waves * 2 * d_state * sizeof(float)};
    size_t at = 0;
    for (int i = 0; i < 8; ++i) {
        p->off[i] = at;
        at += ws_round(sizes[i]);
    }
    p->bytes = (batch > 0 && L > 0) ? at : 0;
    return ok();
}

ssm_status bwd_common(const void *x, const void *dt, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *h0, const void *dy,
                      const float *dh_final, void *dx, void *ddt, void *dz, float *dA, float *dB,
                      float *dC, float *dD, float *dh0, int64_t batch, int64_t L, int64_t d_inner,
                      int32_t d_state, ssm_dtype io, int64_t chunk_len, void *workspace,
                      size_t workspace_bytes, void *hip_stream, const float *states = nullptr) {
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_DTYPE, "io dtype %d unknown", (int)io);
    BwdPlan plan;
    ssm_status st = make_bwd_plan(batch, L, d_inner, d_state, chunk_len, &plan, states != nullptr);
    if (st != SSM_OK) return st;
    if (!A || !D || !dA || !dD) return fail(SSM_ERR_NULL, "A, D, dA and dD are required");
    const bool work = batch > 0 && L > 0;
    if (work && (!x || !dt || !B || !C || !dy || !dx || !ddt || !dB || !dC))
        return fail(SSM_ERR_NULL, "x, dt, B, C, dy, dx, ddt, dB and dC are required");
    if (!aligned(states, 16)) return fail(SSM_ERR_ALIGN, "states must be 16-byte aligned");
    const size_t eb = io_bytes(io);
    if (!aligned(x, eb) || !aligned(dt, eb) || !aligned(z, eb) || !aligned(dy, eb) ||
        !aligned(dx, eb) || !aligned(ddt, eb) || !aligned(dz, eb) || !aligned(B, 4) ||
        !aligned(C, 4) || !aligned(A, 16) || !aligned(D, 4) || !aligned(h0, 16) ||
        !aligned(dh_final, 16) || !aligned(dh0, 16) || !aligned(dA, 4) || !aligned(dB, 4) ||
        !aligned(dC, 4) || !aligned(dD, 4))
        return fail(SSM_ERR_ALIGN, "pointer alignment (A, h0, dh_final, dh0 16 B; B, C, D, dA, dB, dC, dD 4 B; streams element)");
    hipStream_t s = (hipStream_t)hip_stream;
    const int64_t DN = d_inner * d_state;
    if (!work) {  // no steps: dA = dD = 0 and dh0 = dh_final
        st = launch_status(ssm::launch_state_fill(dA, nullptr, DN, s), "fill");
        if (st == SSM_OK) st = launch_status(ssm::launch_state_fill(dD, nullptr, d_inner, s), "fill");
        if (st == SSM_OK && dh0) st = launch_status(ssm::launch_state_fill(dh0, dh_final, batch * DN, s), "fill");
        return st;
    }
    if (!workspace) return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes required", plan.bytes);
    if (workspace_bytes < plan.bytes)
        return fail(SSM_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", workspace_bytes, plan.bytes);
    if (!aligned(workspace, kWsAlign)) return fail(SSM_ERR_ALIGN, "workspace must be 256-byte aligned");
    char *ws = (char *)workspace;
    ssm::ScanArgs f{};
    f.x = x; f.dt = dt; f.B = B; f.C = C; f.z = z; f.A = A; f.D = D; f.h0 = h0;
    f.sumP = (float *)(ws + plan.off[0]);
    f.sumH = (float *)(ws + plan.off[1]);
    f.batch = batch; f.L = L; f.Dn = d_inner;
    f.T = plan.fwd.T; f.n_chunks = plan.fwd.n_chunks;
    f.threads = plan.threads; f.dblocks = plan.dblocks;
    ssm::BwdArgs a{};
    a.x = x; a.dt = dt; a.B = B; a.C = C; a.z = z; a.dy = dy;
    a.A = A; a.D = D; a.h0 = h0; a.dh_final = dh_final;
    a.dx = dx; a.ddt = ddt; a.dz = z ? dz : nullptr;
    a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dh0 = dh0;
    a.sumH = f.sumH;
    a.revQ = (float *)(ws + plan.off[2]);
    a.revG = (float *)(ws + plan.off[3]);
    a.ckpt = states ? const_cast<float *>(states) : (float *)(ws + plan.off[4]);
    a.saved = states != nullptr;
    a.partA = (float *)(ws + plan.off[5]);
    a.partD = (float *)(ws + plan.off[6]);
    a.partBC = (float *)(ws + plan.off[7]);
    a.batch = batch; a.L = L; a.Dn = d_inner; a.T = plan.fwd.T;
    a.n_chunks = plan.fwd.n_chunks; a.dblocks = plan.dblocks; a.threads = plan.threads;
    a.waves = plan.waves;
    a.ck_rows = plan.ck_rows;
    const int iot = io == SSM_BF16 ? 1 : 0;
    return launch_status(ssm::launch_scan_bwd(a, f, iot, d_state, z != nullptr, s), "backward launch");
}

}  // namespace

extern "C" {

size_t ssm_scan_fwd_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state) {
    return ssm_scan_fwd_workspace_ex(batch, L, d_inner, d_state, 0);
}

size_t ssm_scan_fwd_workspace_ex(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                 int64_t chunk_len) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, chunk_len, false, &p, 1,
                  waves_per_simd(Family::Plain)) != SSM_OK)
        return 0;
    return p.ws_bytes;
}

size_t ssm_scan_fwd_c64_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                  int64_t chunk_len) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, chunk_len, true, &p, 1,
                  waves_per_simd(Family::Complex)) != SSM_OK)
        return 0;
    return p.ws_bytes;
}

int64_t ssm_scan_fwd_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, 0, false, &p, 1, waves_per_simd(Family::Plain)) != SSM_OK)
        return 0;
    return p.T;
}

int64_t ssm_scan_fwd_fused_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, 0, false, &p, 1, waves_per_simd(Family::Fused)) != SSM_OK)
        return 0;
    return p.T;
}

int64_t ssm_scan_fwd_c64_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, 0, true, &p, 1, waves_per_simd(Family::Complex)) != SSM_OK)
        return 0;
    return p.T;
}

int64_t ssm_scan_fwd_mimo_chunk_len(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int32_t rank) {
    Plan p;
    if (!valid_rank(rank)) return 0;
    if (make_plan(batch, L, d_inner, d_state, 0, false, &p, rank,
                  waves_per_simd(Family::Mimo, rank)) != SSM_OK)
        return 0;
    return p.T;
}

ssm_status ssm_scan_fwd(const void *x, const void *dt, const float *A, const void *B,
                        const void *C, const float *D, const void *z, const float *h0, void *y,
                        float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                        int32_t d_state, ssm_dtype io, void *workspace, size_t workspace_bytes,
                        void *hip_stream) {
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io, 0,
                       workspace, workspace_bytes, hip_stream, false);
}

ssm_status ssm_scan_fwd_ex(const void *x, const void *dt, const float *A, const void *B,
                           const void *C, const float *D, const void *z, const float *h0, void *y,
                           float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                           int32_t d_state, ssm_dtype io, int64_t chunk_len, void *workspace,
                           size_t workspace_bytes, void *hip_stream) {
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false);
}

ssm_status ssm_scan_fwd_noalloc(const void *x, const void *dt, const float *A, const void *B,
                                const void *C, const float *D, const void *z, const float *h0,
                                void *y, float *h_final, int64_t batch, int64_t L,
                                int64_t d_inner, int32_t d_state, ssm_dtype io,
                                int64_t chunk_len, void *hip_stream) {
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, nullptr, 0, hip_stream, false, nullptr, 0, nullptr, nullptr, 0,
                       true);
}

ssm_status ssm_scan_fwd_c64(const void *x, const void *dt, const float *A, const void *B,
                            const void *C, const float *D, const void *z, const float *h0,
                            void *y, float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                            int32_t d_state, ssm_dtype io, int64_t chunk_len, void *workspace,
                            size_t workspace_bytes, void *hip_stream) {
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, true);
}

ssm_status ssm_scan_fwd_profiled(const void *x, const void *dt, const float *A, const void *B,
                                 const void *C, const float *D, const void *z, const float *h0,
                                 void *y, float *h_final, int64_t batch, int64_t L,
                                 int64_t d_inner, int32_t d_state, ssm_dtype io,
                                 int64_t chunk_len, void *workspace, size_t workspace_bytes,
                                 void *hip_stream, void *const *events, int32_t n_events) {
    if (!events) return fail(SSM_ERR_NULL, "events are required");
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, events, n_events);
}

ssm_status ssm_scan_fwd_c64_profiled(const void *x, const void *dt, const float *A,
                                     const void *B, const void *C, const float *D,
                                     const void *z, const float *h0, void *y, float *h_final,
                                     int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                     ssm_dtype io, int64_t chunk_len, void *workspace,
                                     size_t workspace_bytes, void *hip_stream,
                                     void *const *events, int32_t n_events) {
    if (!events) return fail(SSM_ERR_NULL, "events are required");
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, true, events, n_events);
}

ssm_status ssm_step(float *h, const void *x_t, const void *dt_t, const float *A, const void *B_t,
                    const void *C_t, const float *D, const void *z_t, void *y_t, int64_t n_layers,
                    int64_t n_seq, int64_t d_inner, int32_t d_state, ssm_dtype io,
                    void *hip_stream) {
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, false);
}

ssm_status ssm_step_replay(float *h, const void *x_t, const void *dt_t, const float *A,
                           const void *B_t, const void *C_t, const float *D, const void *z_t,
                           void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                           int32_t d_state, ssm_dtype io, void *hip_stream) {
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, true);
}

ssm_status ssm_step_c64(float *h, const void *x_t, const void *dt_t, const float *A,
                        const void *B_t, const void *C_t, const float *D, const void *z_t,
                        void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                        int32_t d_state, ssm_dtype io, void *hip_stream) {
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, true, false);
}

ssm_status ssm_step_c64_replay(float *h, const void *x_t, const void *dt_t, const float *A,
                               const void *B_t, const void *C_t, const float *D, const void *z_t,
                               void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                               int32_t d_state, ssm_dtype io, void *hip_stream) {
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, true, true);
}

ssm_status ssm_scan_fwd_fused(const void *x_in, const void *dt_raw, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *h0,
                              const float *conv_w, const float *conv_b, int32_t conv_k,
                              const void *conv_state0, void *conv_state_out,
                              const float *dt_bias, void *y, float *h_final, int64_t batch,
                              int64_t L, int64_t d_inner, int32_t d_state, ssm_dtype io,
                              int64_t chunk_len, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
    const InputStage in{conv_w, conv_b, dt_bias, conv_k, conv_state0, conv_state_out};
    return scan_common(x_in, dt_raw, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, nullptr, 0, &in);
}

ssm_status ssm_scan_fwd_fused_save(const void *x_in, const void *dt_raw, const float *A, const void *B,
                                   const void *C, const float *D, const void *z, const float *h0,
                                   const float *conv_w, const float *conv_b, int32_t conv_k,
                                   const void *conv_state0, void *conv_state_out,
                                   const float *dt_bias, void *y, float *h_final, float *states,
                                   void *u_out, void *dt_out, int64_t batch, int64_t L,
                                   int64_t d_inner, int32_t d_state, ssm_dtype io,
                                   int64_t chunk_len, void *workspace, size_t workspace_bytes,
                                   void *hip_stream) {
    if (batch > 0 && L > 0 && (!states || !u_out || !dt_out))
        return fail(SSM_ERR_NULL, "states, u_out and dt_out are required");
    const size_t eb = io == SSM_BF16 ? 2 : 4;
    if (!aligned(u_out, eb) || !aligned(dt_out, eb))
        return fail(SSM_ERR_ALIGN, "u_out and dt_out must be element-aligned");
    // The rescan writes a chunk's u and dt while other chunks still read x_in, dt_raw
    // and write y.
    const size_t rows = (size_t)(batch > 0 && L > 0 && d_inner > 0 ? batch * L * d_inner : 0) * eb;
    const void *ins[] = {x_in, dt_raw, y};
    for (const void *p : ins)
        if (overlaps(u_out, rows, p, rows) || overlaps(dt_out, rows, p, rows))
            return fail(SSM_ERR_UNSUPPORTED, "u_out and dt_out must not overlap x_in, dt_raw or y");
    if (overlaps(u_out, rows, dt_out, rows))
        return fail(SSM_ERR_UNSUPPORTED, "u_out and dt_out must not overlap");
    InputStage in{conv_w, conv_b, dt_bias, conv_k, conv_state0, conv_state_out};
    in.u_out = u_out;
    in.dt_out = dt_out;
    return scan_common(x_in, dt_raw, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, nullptr, 0, &in,
                       nullptr, 0, false, batch > 0 && L > 0 ? states : nullptr);
}

ssm_status ssm_scan_fwd_fused_profiled(const void *x_in, const void *dt_raw, const float *A,
                                       const void *B, const void *C, const float *D,
                                       const void *z, const float *h0, const float *conv_w,
                                       const float *conv_b, int32_t conv_k,
                                       const void *conv_state0, void *conv_state_out,
                                       const float *dt_bias, void *y, float *h_final,
                                       int64_t batch, int64_t L, int64_t d_inner,
                                       int32_t d_state, ssm_dtype io, int64_t chunk_len,
                                       void *workspace, size_t workspace_bytes, void *hip_stream,
                                       void *const *events, int32_t n_events) {
    if (!events) return fail(SSM_ERR_NULL, "events are required");
    const InputStage in{conv_w, conv_b, dt_bias, conv_k, conv_state0, conv_state_out};
    return scan_common(x_in, dt_raw, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, events, n_events,
                       &in);
}

ssm_status ssm_step_fused(float *h, void *conv_state, const void *x_t, const void *dt_t,
                          const float *A, const void *B_t, const void *C_t, const float *D,
                          const void *z_t, const float *conv_w, const float *conv_b,
                          int32_t conv_k, const float *dt_bias, void *y_t, int64_t n_layers,
                          int64_t n_seq, int64_t d_inner, int32_t d_state, ssm_dtype io,
                          void *hip_stream) {
    const InputStage in{conv_w, conv_b, dt_bias, conv_k, nullptr, conv_state};
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, false, &in);
}

ssm_status ssm_step_fused_replay(float *h, void *conv_state, const void *x_t, const void *dt_t,
                                 const float *A, const void *B_t, const void *C_t, const float *D,
                                 const void *z_t, const float *conv_w, const float *conv_b,
                                 int32_t conv_k, const float *dt_bias, void *y_t,
                                 int64_t n_layers, int64_t n_seq, int64_t d_inner,
                                 int32_t d_state, ssm_dtype io, void *hip_stream) {
    const InputStage in{conv_w, conv_b, dt_bias, conv_k, nullptr, conv_state};
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, true, &in);
}

ssm_status ssm_scan_fwd_trap(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             const void *x_prev, const void *B_prev, const void *lam, void *y,
                             float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                             int32_t d_state, ssm_dtype io, int64_t chunk_len, void *workspace,
                             size_t workspace_bytes, void *hip_stream) {
    const Trap tr{x_prev, B_prev, lam};
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, nullptr, 0,
                       nullptr, &tr);
}

ssm_status ssm_scan_fwd_trap_profiled(const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *h0, const void *x_prev,
                                      const void *B_prev, const void *lam, void *y,
                                      float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                                      int32_t d_state, ssm_dtype io, int64_t chunk_len,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *const *events, int32_t n_events) {
    if (!events) return fail(SSM_ERR_NULL, "events are required");
    const Trap tr{x_prev, B_prev, lam};
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, events, n_events,
                       nullptr, &tr);
}

ssm_status ssm_step_trap(float *h, const void *x_prev, const void *B_prev, const void *x_t,
                         const void *dt_t, const void *lam_t, const float *A, const void *B_t,
                         const void *C_t, const float *D, const void *z_t, void *y_t,
                         int64_t n_layers, int64_t n_seq, int64_t d_inner, int32_t d_state,
                         ssm_dtype io, void *hip_stream) {
    const Trap tr{x_prev, B_prev, lam_t};
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, false, nullptr, &tr);
}

ssm_status ssm_step_trap_replay(float *h, const void *x_prev, const void *B_prev,
                                const void *x_t, const void *dt_t, const void *lam_t,
                                const float *A, const void *B_t, const void *C_t, const float *D,
                                const void *z_t, void *y_t, int64_t n_layers, int64_t n_seq,
                                int64_t d_inner, int32_t d_state, ssm_dtype io,
                                void *hip_stream) {
    const Trap tr{x_prev, B_prev, lam_t};
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, true, nullptr, &tr);
}

size_t ssm_scan_fwd_mimo_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                   int32_t rank, int64_t chunk_len) {
    Plan p;
    if (!valid_rank(rank)) return 0;
    if (make_plan(batch, L, d_inner, d_state, chunk_len, false, &p, rank,
                  waves_per_simd(Family::Mimo, rank)) != SSM_OK)
        return 0;
    return p.ws_bytes;
}

ssm_status ssm_scan_fwd_mimo(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             void *y, float *h_final, int64_t batch, int64_t L, int64_t d_inner,
                             int32_t d_state, int32_t rank, ssm_dtype io, int64_t chunk_len,
                             void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (rank == 0) return fail(SSM_ERR_UNSUPPORTED, "rank 0 not in {1,2,4,8}");
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, nullptr, 0,
                       nullptr, nullptr, rank);
}

ssm_status ssm_scan_fwd_mimo_profiled(const void *x, const void *dt, const float *A,
                                      const void *B, const void *C, const float *D,
                                      const void *z, const float *h0, void *y, float *h_final,
                                      int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                      int32_t rank, ssm_dtype io, int64_t chunk_len,
                                      void *workspace, size_t workspace_bytes, void *hip_stream,
                                      void *const *events, int32_t n_events) {
    if (!events) return fail(SSM_ERR_NULL, "events are required");
    if (rank == 0) return fail(SSM_ERR_UNSUPPORTED, "rank 0 not in {1,2,4,8}");
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, events, n_events,
                       nullptr, nullptr, rank);
}

ssm_status ssm_step_mimo(float *h, const void *x_t, const void *dt_t, const float *A,
                         const void *B_t, const void *C_t, const float *D, const void *z_t,
                         void *y_t, int64_t n_layers, int64_t n_seq, int64_t d_inner,
                         int32_t d_state, int32_t rank, ssm_dtype io, void *hip_stream) {
    if (rank == 0) return fail(SSM_ERR_UNSUPPORTED, "rank 0 not in {1,2,4,8}");
    return step_common(h, x_t, dt_t, A, B_t, C_t, D, z_t, y_t, n_layers, n_seq, d_inner, d_state,
                       io, hip_stream, false, false, nullptr, nullptr, rank);
}

size_t ssm_scan_bwd_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                              int64_t chunk_len) {
    BwdPlan p;
    if (make_bwd_plan(batch, L, d_inner, d_state, chunk_len, &p) != SSM_OK) return 0;
    return p.bytes;
}

ssm_status ssm_scan_bwd(const void *x, const void *dt, const float *A, const void *B, const void *C,
                        const float *D, const void *z, const float *h0, const void *dy,
                        const float *dh_final, void *dx, void *ddt, void *dz, float *dA, float *dB,
                        float *dC, float *dD, float *dh0, int64_t batch, int64_t L,
                        int64_t d_inner, int32_t d_state, ssm_dtype io, int64_t chunk_len,
                        void *workspace, size_t workspace_bytes, void *hip_stream) {
    return bwd_common(x, dt, A, B, C, D, z, h0, dy, dh_final, dx, ddt, dz, dA, dB, dC, dD, dh0,
                      batch, L, d_inner, d_state, io, chunk_len, workspace, workspace_bytes,
                      hip_stream);
}

size_t ssm_scan_fwd_save_states_bytes(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state) {
    if (batch < 0 || L < 0 || d_inner < 1 || !valid_state(d_state)) return 0;
    const int64_t rows = (L + ssm::kStateEvery - 1) / ssm::kStateEvery;
    return (size_t)rows * (size_t)batch * (size_t)d_inner * (size_t)d_state * sizeof(float);
}

size_t ssm_scan_fwd_save_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                   int64_t chunk_len) {
    Plan p;
    if (make_plan(batch, L, d_inner, d_state, chunk_len, false, &p, 1, waves_per_simd(Family::Plain),
                  ssm::kStateEvery) != SSM_OK)
        return 0;
    return p.ws_bytes;
}

ssm_status ssm_scan_fwd_save(const void *x, const void *dt, const float *A, const void *B,
                             const void *C, const float *D, const void *z, const float *h0,
                             void *y, float *h_final, float *states, int64_t batch, int64_t L,
                             int64_t d_inner, int32_t d_state, ssm_dtype io, int64_t chunk_len,
                             void *workspace, size_t workspace_bytes, void *hip_stream) {
    if (batch > 0 && L > 0 && !states) return fail(SSM_ERR_NULL, "states is required");
    return scan_common(x, dt, A, B, C, D, z, h0, y, h_final, batch, L, d_inner, d_state, io,
                       chunk_len, workspace, workspace_bytes, hip_stream, false, nullptr, 0,
                       nullptr, nullptr, 0, false, batch > 0 && L > 0 ? states : nullptr);
}

size_t ssm_scan_bwd_saved_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int64_t chunk_len) {
    BwdPlan p;
    if (make_bwd_plan(batch, L, d_inner, d_state, chunk_len, &p, true) != SSM_OK) return 0;
    return p.bytes;
}

ssm_status ssm_scan_bwd_saved(const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *states,
                              const void *dy, const float *dh_final, void *dx, void *ddt, void *dz,
                              float *dA, float *dB, float *dC, float *dD, float *dh0, int64_t batch,
                              int64_t L, int64_t d_inner, int32_t d_state, ssm_dtype io,
                              int64_t chunk_len, void *workspace, size_t workspace_bytes,
                              void *hip_stream) {
    if (batch > 0 && L > 0 && !states) return fail(SSM_ERR_NULL, "states is required");
    return bwd_common(x, dt, A, B, C, D, z, nullptr, dy, dh_final, dx, ddt, dz, dA, dB, dC, dD, dh0,
                      batch, L, d_inner, d_state, io, chunk_len, workspace, workspace_bytes,
                      hip_stream, batch > 0 && L > 0 ? states : nullptr);
}

// ---------------------------------------------------------------- backward through the input stage
// The two streaming kernels of the input stage take chunks of their own (independent:
// enough for about 8 blocks of 256 channels per SIMD, 8192 on 256 CUs, i.e. 2 blocks of
// 256 lanes per SIMD at four channels per lane, chunks of at least 128 steps). Workspace: the scan backward's, then u, dt, du, ddt
// ([batch][L][d_inner] of io each; u and dt only when they are made here, not given by
// the fused training forward) and the partial sums ([n][batch][d_inner][conv_k + 2]
// fp32), each 256-byte aligned.
struct InBwdPlan {
    int64_t T;
    int32_t n_chunks;
    int32_t nbuf;  // io buffers in the workspace: 4 (u, dt, du, ddt) or 2 (du, ddt)
    size_t scan_ws, buf, part, bytes;
};

ssm_status make_in_bwd_plan(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                            int32_t conv_k, ssm_dtype io, int64_t chunk_len, InBwdPlan *p,
                            bool saved = false) {
    if (io != SSM_F32 && io != SSM_BF16) return fail(SSM_ERR_DTYPE, "io dtype %d unknown", (int)io);
    if (conv_k < 0 || conv_k > 4) return fail(SSM_ERR_UNSUPPORTED, "conv_k %d not in 0..4", conv_k);
    BwdPlan bp;
    const ssm_status st = make_bwd_plan(batch, L, d_inner, d_state, chunk_len, &bp, saved);
    if (st != SSM_OK) return st;
    const int64_t blocks = std::max<int64_t>(1, batch * ((d_inner + 255) / 256));
    const int64_t want = 8 * device_simds();
    int64_t n = std::min<int64_t>((want + blocks - 1) / blocks, std::max<int64_t>(1, L / 128));
    n = std::max<int64_t>(n, 1);
    p->T = L > 0 ? (L + n - 1) / n : 1;
    p->n_chunks = L > 0 ? (int32_t)((L + p->T - 1) / p->T) : 0;
    p->scan_ws = ws_round(bp.bytes);
    p->buf = ws_round((size_t)batch * (size_t)L * (size_t)d_inner * io_bytes(io));
    p->part = ws_round((size_t)p->n_chunks * (size_t)batch * (size_t)d_inner * (size_t)(conv_k + 2) * sizeof(float));
    p->nbuf = saved ? 2 : 4;
    p->bytes = p->scan_ws + (size_t)p->nbuf * p->buf + p->part;
    return ok();
}

size_t ssm_scan_bwd_fused_workspace(int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                                    int32_t conv_k, ssm_dtype io, int64_t chunk_len) {
    InBwdPlan p;
    if (make_in_bwd_plan(batch, L, d_inner, d_state, conv_k, io, chunk_len, &p) != SSM_OK) return 0;
    return p.bytes;
}

namespace {
ssm_status bwd_fused_common(const void *x_in, const void *dt_raw, const float *A, const void *B,
                            const void *C, const float *D, const void *z, const float *h0,
                            const float *states, const void *u_saved, const void *dt_saved,
                            const float *conv_w, const float *conv_b,
                            int32_t conv_k, const void *conv_state0, const float *dt_bias,
                            const void *dy, const float *dh_final, void *dx_in, void *ddt_raw,
                            void *dz, float *dA, float *dB, float *dC, float *dD, float *dh0,
                            float *dconv_w, float *dconv_b, float *ddt_bias, void *dconv_state0,
                            int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                            ssm_dtype io, int64_t chunk_len, void *workspace,
                            size_t workspace_bytes, void *hip_stream, bool saved) {
    InBwdPlan p;
    ssm_status st = make_in_bwd_plan(batch, L, d_inner, d_state, conv_k, io, chunk_len, &p, saved);
    if (st != SSM_OK) return st;
    const size_t eb = io_bytes(io);
    st = check_input_stage(InputStage{conv_w, conv_b, dt_bias, conv_k, conv_state0, dconv_state0}, eb);
    if (st != SSM_OK) return st;
    if (conv_k > 0 && !dconv_w) return fail(SSM_ERR_NULL, "dconv_w is required when conv_k > 0");
    const bool work = batch > 0 && L > 0;
    if (work && (!x_in || !dt_raw || !dx_in || !ddt_raw))
        return fail(SSM_ERR_NULL, "x_in, dt_raw, dx_in and ddt_raw are required");
    if (saved && work && (!states || !u_saved || !dt_saved))
        return fail(SSM_ERR_NULL, "states, u and dt are required");
    if (!aligned(states, 16)) return fail(SSM_ERR_ALIGN, "states must be 16-byte aligned");
    if (!aligned(u_saved, eb) || !aligned(dt_saved, eb))
        return fail(SSM_ERR_ALIGN, "u and dt must be element-aligned");
    if (!aligned(x_in, eb) || !aligned(dt_raw, eb) || !aligned(dx_in, eb) || !aligned(ddt_raw, eb) ||
        !aligned(dconv_w, 4) || !aligned(dconv_b, 4) || !aligned(ddt_bias, 4))
        return fail(SSM_ERR_ALIGN, "pointer alignment (x_in, dt_raw, dx_in, ddt_raw element; dconv_w, dconv_b, ddt_bias 4 B)");
    const size_t rows = (size_t)batch * (size_t)L * (size_t)d_inner * eb;
    if (overlaps(dx_in, rows, x_in, rows))
        return fail(SSM_ERR_UNSUPPORTED, "dx_in must not overlap x_in (a chunk reads the inputs after it)");
    if (saved) {
        // the scan's backward reads u and dt while it writes dz and the input stage's
        // backward writes dx_in and ddt_raw
        const void *outs[] = {dx_in, ddt_raw, dz};
        for (const void *o : outs)
            if (overlaps(u_saved, rows, o, rows) || overlaps(dt_saved, rows, o, rows))
                return fail(SSM_ERR_UNSUPPORTED, "u and dt must not overlap dx_in, ddt_raw or dz");
    }
    if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes))
        return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed", p.bytes);
    if (!aligned(workspace, kWsAlign)) return fail(SSM_ERR_ALIGN, "workspace must be 256-byte aligned");
    char *ws = (char *)workspace;
    ssm::InBwdArgs a{};
    a.x_in = x_in; a.dt_raw = dt_raw;
    a.conv_w = conv_k > 0 ? conv_w : nullptr; a.conv_b = conv_k > 0 ? conv_b : nullptr;
    a.dt_bias = dt_bias; a.conv_state0 = conv_k > 1 ? conv_state0 : nullptr;
    // u and dt: from the fused training forward, or made here from x_in and dt_raw
    char *io_bufs = ws ? ws + p.scan_ws : nullptr;
    a.u = saved ? const_cast<void *>(u_saved) : io_bufs;
    a.dt = saved ? const_cast<void *>(dt_saved) : (ws ? io_bufs + p.buf : nullptr);
    a.du = ws ? io_bufs + (size_t)(p.nbuf - 2) * p.buf : nullptr;
    a.ddt = ws ? io_bufs + (size_t)(p.nbuf - 1) * p.buf : nullptr;
    a.dx_in = dx_in; a.ddt_raw = ddt_raw;
    a.dconv_state0 = conv_k > 1 ? dconv_state0 : nullptr;
    a.part = ws ? (float *)(io_bufs + (size_t)p.nbuf * p.buf) : nullptr;
    a.dconv_w = conv_k > 0 ? dconv_w : nullptr; a.dconv_b = conv_k > 0 ? dconv_b : nullptr;
    a.ddt_bias = ddt_bias;
    a.batch = batch; a.L = L; a.Dn = d_inner; a.T = p.T; a.n_chunks = p.n_chunks; a.conv_k = conv_k;
    hipStream_t s = (hipStream_t)hip_stream;
    const int iot = io == SSM_BF16 ? 1 : 0;
    if (work && !saved) {
        st = launch_status(ssm::launch_input_fwd(a, iot, s), "input stage (forward)");
        if (st != SSM_OK) return st;
    }
    st = bwd_common(a.u, a.dt, A, B, C, D, z, saved ? nullptr : h0, dy, dh_final, const_cast<void *>(a.du),
                    const_cast<void *>(a.ddt), dz, dA, dB, dC, dD, dh0, batch, L, d_inner, d_state,
                    io, chunk_len, ws, p.scan_ws, hip_stream, saved && work ? states : nullptr);
    if (st != SSM_OK) return st;
    if (work) return launch_status(ssm::launch_input_bwd(a, iot, s), "input stage (backward)");
    // no steps: the input stage's own gradients are zero
    const int64_t Kw = conv_k > 0 ? conv_k : 0;
    const struct { void *p; int64_t n; int eb; } zero[] = {
        {a.dconv_w, d_inner * Kw, 4}, {a.dconv_b, d_inner, 4}, {a.ddt_bias, d_inner, 4},
        {a.dconv_state0, batch * (conv_k > 1 ? conv_k - 1 : 0) * d_inner, (int)eb}};
    for (const auto &zf : zero) {
        if (!zf.p || zf.n <= 0) continue;
        st = launch_status(ssm::launch_elem_fill(zf.p, nullptr, zf.n, zf.eb, s), "zero fill");
        if (st != SSM_OK) return st;
    }
    return ok();
}
}  // namespace

ssm_status ssm_scan_bwd_fused(const void *x_in, const void *dt_raw, const float *A, const void *B,
                              const void *C, const float *D, const void *z, const float *h0,
                              const float *conv_w, const float *conv_b, int32_t conv_k,
                              const void *conv_state0, const float *dt_bias, const void *dy,
                              const float *dh_final, void *dx_in, void *ddt_raw, void *dz,
                              float *dA, float *dB, float *dC, float *dD, float *dh0,
                              float *dconv_w, float *dconv_b, float *ddt_bias, void *dconv_state0,
                              int64_t batch, int64_t L, int64_t d_inner, int32_t d_state,
                              ssm_dtype io, int64_t chunk_len, void *workspace,
                              size_t workspace_bytes, void *hip_stream) {
    return bwd_fused_common(x_in, dt_raw, A, B, C, D, z, h0, nullptr, nullptr, nullptr, conv_w, conv_b, conv_k,
                            conv_state0, dt_bias, dy, dh_final, dx_in, ddt_raw, dz, dA, dB, dC, dD,
                            dh0, dconv_w, dconv_b, ddt_bias, dconv_state0, batch, L, d_inner,
                            d_state, io, chunk_len, workspace, workspace_bytes, hip_stream, false);
}

size_t ssm_scan_bwd_fused_saved_workspace(int64_t batch, int64_t L, int64_t d_inner,
                                          int32_t d_state, int32_t conv_k, ssm_dtype io,
                                          int64_t chunk_len) {
    InBwdPlan p;
    if (make_in_bwd_plan(batch, L, d_inner, d_state, conv_k, io, chunk_len, &p, true) != SSM_OK) return 0;
    return p.bytes;
}

ssm_status ssm_scan_bwd_fused_saved(const void *x_in, const void *dt_raw, const float *A,
                                    const void *B, const void *C, const float *D, const void *z,
                                    const float *states, const void *u, const void *dt,
                                    const float *conv_w, const float *conv_b,
                                    int32_t conv_k, const void *conv_state0, const float *dt_bias,
                                    const void *dy, const float *dh_final, void *dx_in,
                                    void *ddt_raw, void *dz, float *dA, float *dB, float *dC,
                                    float *dD, float *dh0, float *dconv_w, float *dconv_b,
                                    float *ddt_bias, void *dconv_state0, int64_t batch, int64_t L,
                                    int64_t d_inner, int32_t d_state, ssm_dtype io,
                                    int64_t chunk_len, void *workspace, size_t workspace_bytes,
                                    void *hip_stream) {
    return bwd_fused_common(x_in, dt_raw, A, B, C, D, z, nullptr, states, u, dt, conv_w, conv_b, conv_k,
                            conv_state0, dt_bias, dy, dh_final, dx_in, ddt_raw, dz, dA, dB, dC, dD,
                            dh0, dconv_w, dconv_b, ddt_bias, dconv_state0, batch, L, d_inner,
                            d_state, io, chunk_len, workspace, workspace_bytes, hip_stream, true);
}

const char *ssm_status_str(ssm_status s) {
    switch (s) {
        case SSM_OK: return "ok";
        case SSM_ERR_NULL: return "required pointer is NULL";
        case SSM_ERR_SHAPE: return "invalid size";
        case SSM_ERR_DTYPE: return "invalid io dtype";
        case SSM_ERR_ALIGN: return "misaligned pointer";
        case SSM_ERR_UNSUPPORTED: return "unsupported d_state, chunk length, conv_k or overlap";
        case SSM_ERR_WORKSPACE: return "workspace missing or too small";
        case SSM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *ssm_last_error(void) { return g_err; }

int32_t ssm_abi_version(void) { return 3; }

}  // extern "C"
