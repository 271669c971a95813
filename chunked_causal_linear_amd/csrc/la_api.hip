// liblinattn C ABI: argument checks, planning (tile sizes, groups, workspace)
// and launches.  Every entry point validates everything before it enqueues
// anything, never allocates, never synchronises, and never throws.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/la.h"
#include "la_chunked_bf16.hpp"
#include "la_kernels.hpp"

#ifndef LA_PIPE_TARGET
#define LA_PIPE_TARGET 256
#endif

namespace la {
hipError_t fwd_pipe_bf16(const FwdParams& p, int DK, int DVT, int C, int64_t grid, hipStream_t s);
}

namespace {

thread_local char g_last_error[512] = "";

la_status fail(la_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

la_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return LA_OK;
    return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2_in(int64_t x, int64_t lo, int64_t hi) {
    if (x < lo || x > hi) return false;
    return (x & (x - 1)) == 0;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// tile choices
// ---------------------------------------------------------------------------
int kernel_dk_bf16(int64_t dk) { return dk <= 32 ? 32 : (int)dk; }
int kernel_dk_i8(int64_t dk) { return dk <= 64 ? 64 : (int)dk; }
int kernel_dvt(int64_t dv) { return dv >= 64 ? 64 : (int)dv; }

// largest row tile compiled for (DK, DVT); the hi/lo split of phi(K) (elu+1
// in the kernel) needs one more K^T tile of LDS
int max_tile_bf16(int DK, int DVT, bool split) {
    if (DK <= 64) return 128;
    if (DK == 128) return (DVT == 16 || split) ? 64 : 128;
    return DVT == 16 ? 32 : 64;  // DK == 256
}

int tile_bf16(int64_t C, int DK, int DVT, bool split) {
    int T = C <= 32 ? 32 : (C <= 64 ? 64 : 128);
    const int tmax = max_tile_bf16(DK, DVT, split);
    return T < tmax ? T : tmax;
}

int tile_i8(int64_t C, int DK, int DVT) {
    const bool has128 = (DK == 64) || (DK == 128 && DVT == 64);
    return (C > 64 && has128) ? 128 : 64;
}

// ---------------------------------------------------------------------------
// forward plan
// ---------------------------------------------------------------------------
struct Plan {
    bool i8;
    int64_t BH, L, C, dk, dv, d_in;
    int64_t n_chunks, G, n_groups;
    int DK, DVT, T, n_dvt;
    bool premap;  // phi computed by a separate pass into the workspace
    bool favor;   // FAVOR+ mapped inside the streaming kernels (no mapped copies)
    bool pipe;    // streaming phase-3 kernel (chunks of 32, 64 or 128 rows)
    bool causal, normalize;
    int64_t sub;       // phase-1 states per group (finer grain than the groups when they are few and long)
    bool final_from_scan;  // a returned final state / normaliser is the scan's total, not phase 3's
    size_t ws_phi;     // bytes of one mapped q or k copy
    size_t ws_states;  // bytes of the group states
    size_t ws_z;
    size_t ws_total;
};

la_status check_dtypes_forward(la_dtype in_dt, la_dtype out_dt, int normalize, la_fmap f, float in_scale) {
    if (in_dt == LA_BF16) {
        if (out_dt != LA_BF16 && out_dt != LA_F32)
            return fail(LA_ERR_UNSUPPORTED, "bf16 inputs need an LA_BF16 or LA_F32 output");
        return LA_OK;
    }
    if (in_dt == LA_I8) {
        if (normalize) return fail(LA_ERR_UNSUPPORTED, "the int8 path has no normaliser");
        if (in_scale != 1.0f) return fail(LA_ERR_UNSUPPORTED, "the int8 path has no input scale");
        if (f != LA_FMAP_IDENTITY) return fail(LA_ERR_UNSUPPORTED, "the int8 path has no feature map");
        if (out_dt != LA_I32) return fail(LA_ERR_UNSUPPORTED, "int8 inputs need an LA_I32 output");
        return LA_OK;
    }
    return fail(LA_ERR_UNSUPPORTED, "input type must be LA_BF16 or LA_I8");
}

la_status make_plan(Plan& P, la_dtype in_dt, int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                    int causal, int normalize, la_fmap f, int64_t m, float in_scale, int64_t group,
                    bool decay, bool bf16_out = false) {
    if (BH < 1 || L < 1 || d_in < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (f != LA_FMAP_IDENTITY && f != LA_FMAP_ELU1 && f != LA_FMAP_FAVOR)
        return fail(LA_ERR_INVALID_ARG, "unknown feature map %d", (int)f);
    if (!(in_scale == in_scale)) return fail(LA_ERR_INVALID_ARG, "in_scale is NaN");
    P.i8 = in_dt == LA_I8;
    P.BH = BH;
    P.L = L;
    P.d_in = d_in;
    P.dv = d_v;
    P.causal = causal != 0;
    P.normalize = normalize != 0;
    P.dk = f == LA_FMAP_FAVOR ? m : d_in;
    if (f == LA_FMAP_FAVOR) {
        if (!pow2_in(m, 16, 256)) return fail(LA_ERR_UNSUPPORTED, "FAVOR+ feature count m must be 16..256, a power of two");
        if (!pow2_in(d_in, 16, 128)) return fail(LA_ERR_UNSUPPORTED, "FAVOR+ input width must be 16..128, a power of two");
    }
    if (!pow2_in(P.dk, 16, 256)) return fail(LA_ERR_UNSUPPORTED, "feature width d_k=%lld unsupported (16..256, power of two)", (long long)P.dk);
    if (!pow2_in(d_v, 16, 256)) return fail(LA_ERR_UNSUPPORTED, "value width d_v=%lld unsupported (16..256, power of two)", (long long)d_v);
    if (BH * L > ((int64_t)1 << 40)) return fail(LA_ERR_UNSUPPORTED, "problem too large");

    int64_t Ce = C <= 0 ? 1 : C;
    if (Ce > L) Ce = L;  // one chunk
    // FAVOR+ maps q and k in a separate pass; elu+1 is applied in the kernels
    // (on load, or to the landed tiles); the identity map with a scale s runs
    // unscaled and scales the results (outputs by s^2 unless normalised, the
    // final state by s), which is exact.
    P.DVT = kernel_dvt(d_v);
    P.n_dvt = (int)(d_v / P.DVT);
    if (P.i8) {
        P.DK = kernel_dk_i8(P.dk);
    } else {
        P.DK = kernel_dk_bf16(P.dk);
    }

    // The streaming kernel covers chunks of 32, 64 or 128 rows at feature
    // widths 64 and 128, with or without the normaliser, for every map (elu+1
    // applied in the kernel, FAVOR+ beforehand).  It fills the LDS and runs one
    // workgroup per CU.  With a map it sums bf16(phi(k)) into its state; a
    // returned final state then comes from phase 1 (which adds phi(k)'s
    // residual) and the scan's total.
    // At width 256 (FAVOR+ with 256 features) it takes 32 value columns per
    // workgroup and chunks of 32 or 64 (two 68 KB stages).
    P.pipe = !P.i8 && P.causal &&
             (((Ce == 32 || Ce == 64 || Ce == 128) && d_v % 64 == 0 && (P.dk == 64 || P.dk == 128)) ||
              ((Ce == 32 || Ce == 64) && d_v % 32 == 0 && P.dk == 256));
    // FAVOR+ with 64 input features, 64, 128 or 256 random features, chunks
    // of 64 rows, value columns a multiple of 64 and a bf16 output: the
    // streaming kernels map q and k themselves from W held in LDS
    // (la_favor.hip), so the mapped copies never go through memory.
    P.favor = !P.i8 && P.causal && f == LA_FMAP_FAVOR && bf16_out && !decay && d_in == 64 &&
              (m == 64 || m == 128 || m == 256) && Ce == 64 && d_v % 64 == 0;
    if (P.favor) P.pipe = true;
    P.final_from_scan = P.pipe && f != LA_FMAP_IDENTITY;
    P.premap = f == LA_FMAP_FAVOR && !P.favor;
    if (P.pipe) {
        P.DK = (int)P.dk;
        P.DVT = (P.dk == 256 && !P.favor) ? 32 : 64;
        P.n_dvt = (int)(d_v / P.DVT);
    }

    if (!P.causal) {
        // total state from one chunk of L rows, then every tile reads it
        P.T = 64;
        if (!P.i8 && P.T > max_tile_bf16(P.DK, P.DVT, false)) P.T = max_tile_bf16(P.DK, P.DVT, false);
        P.C = P.T;
        P.n_chunks = cdiv(L, P.C);
        P.G = 1;
        P.n_groups = P.n_chunks;
    } else {
        P.C = Ce;
        P.T = P.i8 ? tile_i8(Ce, P.DK, P.DVT) : tile_bf16(Ce, P.DK, P.DVT, f == LA_FMAP_ELU1);
        P.n_chunks = cdiv(L, Ce);
        if (group > 0) {
            P.G = group < P.n_chunks ? group : P.n_chunks;
        } else {
            // enough workgroups for the 256 compute units: four per CU over the
            // launch when two fit at once (the kernels without the hi/lo split
            // run two per CU), one per CU otherwise; fewer groups mean less
            // phase-1 traffic, more mean more loads in flight per CU.  The
            // int8 kernel runs two per CU: two per CU over the launch
            // (measured best: 0.48 ms at 128 heads x 8192 rows, against 0.63
            // with one group per head and 0.51 with four).  The streaming
            // kernel holds a CU alone, so it gets at most one workgroup per CU
            // (a second partial round would double the time of the CUs that
            // run it).
            const bool split = f == LA_FMAP_ELU1 || f == LA_FMAP_FAVOR;
            const int64_t target = P.pipe ? LA_PIPE_TARGET : (P.i8 ? 512 : (split ? 256 : 1024));
            const int64_t base = BH * P.n_dvt;
            int64_t want = base >= target ? 1 : (P.pipe ? target / base : cdiv(target, base));
            if (want > P.n_chunks) want = P.n_chunks;
            P.G = cdiv(P.n_chunks, want);
        }
        // chunks of 32 are walked in tiles of two: groups start on a tile.  An
        // odd group the caller asked for goes to the general kernel, except
        // with the decay, which only the streaming kernel has: rounded up
        // there (the group size changes no result beyond rounding order).
        if (P.pipe && Ce == 32 && P.G < P.n_chunks && (P.G & 1)) {
            if (group > 0 && !decay)
                P.pipe = false;
            else
                P.G += 1;
        }
        P.n_groups = cdiv(P.n_chunks, P.G);
    }
    if (!P.pipe && !P.i8 && P.causal && P.DVT != kernel_dvt(d_v)) {
        P.DVT = kernel_dvt(d_v);
        P.n_dvt = (int)(d_v / P.DVT);
    }
    const int64_t grid = BH * P.n_groups * P.n_dvt;
    if (grid > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");

    // Phase 1 sums each group's rows; a few long groups would leave most CUs
    // idle, so each group's rows are split into `sub` equal pieces (of >= 512
    // rows, each reading >= 8x the state it writes); the scan then walks the
    // pieces and group g starts from the prefix at piece g * sub.  The
    // register-staged phase-1 kernel runs several workgroups per CU: pieces
    // double while fewer than 1024 run.  The streaming one (bf16 at feature
    // width 64, 128 or 256, value columns a multiple of 64, pieces of whole
    // 64-row tiles, K plain or pre-mapped) holds a CU alone: pieces
    // double while the workgroups still fit the CUs in one round.  With elu+1
    // applied in phase 1 it runs two workgroups per CU and its pieces are
    // planned like the register-staged kernel's (measured best).
    P.sub = 1;
    const int64_t n_summed = P.final_from_scan ? P.n_groups : P.n_groups - 1;  // groups phase 1 may sum
    if (P.causal && n_summed > 0) {
        const int64_t n_dvt1 = d_v / kernel_dvt(d_v);
        // a piece reads at least eight times the state it writes
        const int64_t min_rows = std::max<int64_t>(512, cdiv(16 * P.dk * d_v, P.dk + d_v));
        const bool stream1 = !P.i8 && f != LA_FMAP_ELU1 && (P.dk == 64 || P.dk == 128 || P.dk == 256) &&
                             d_v % 64 == 0 && (P.G * P.C) % 64 == 0;
        auto more = [&]() {
            const int64_t rows = P.G * P.C / (2 * P.sub);
            if ((P.G * P.C) % (2 * P.sub) != 0 || rows < min_rows) return false;
            if (stream1) return rows % 64 == 0 && 2 * BH * n_summed * P.sub * n_dvt1 <= 256;
            return BH * n_summed * P.sub * n_dvt1 < 1024;
        };
        while (more()) P.sub *= 2;
    }

    const size_t st_elem = 4;
    P.ws_phi = P.premap ? align256((size_t)BH * L * P.dk * 2) : 0;
    const int64_t n_state_slots =
        P.causal ? ((P.n_groups > 1 || P.final_from_scan) ? P.n_groups * P.sub : 0) : 1;
    P.ws_states = align256((size_t)BH * n_state_slots * P.dk * d_v * st_elem);
    P.ws_z = (P.normalize && n_state_slots) ? align256((size_t)BH * n_state_slots * P.dk * st_elem) : 0;
    if (n_state_slots == 0) P.ws_states = 0;
    // pre-mapped: phi(q), phi(k) and the bf16 residual of phi(k) (the state
    // sums use hi + lo, so the bf16 rounding of phi does not accumulate over L)
    P.ws_total = 3 * P.ws_phi + P.ws_states + P.ws_z;
    return LA_OK;
}

bool xcd_ok(int64_t grid) { return grid >= 8 && grid % 8 == 0; }

}  // namespace

// Phase 3 for a planned call: the fused output kernel over every (head,
// group, column tile), starting each group from its prefix state.
static la_status launch_phase3(const Plan& P, const void* qm, const void* km, const void* klo, const void* v,
                               void* o, la_dtype out_dt, const void* states, const void* zst, void* S_final,
                               void* z_final, int fmap_in_kernel, float in_scale, bool scaled_identity,
                               hipStream_t s, float lg = 0.0f) {
    const int64_t BH = P.BH, L = P.L, d_v = P.dv;
    const int64_t grid = BH * P.n_groups * P.n_dvt;
    if (P.i8) {
        la::FwdParamsI8 p{};
        p.q = static_cast<const signed char*>(qm);
        p.k = static_cast<const signed char*>(km);
        p.v = static_cast<const signed char*>(v);
        p.o = static_cast<int*>(o);
        p.P0 = static_cast<const int*>(states);
        p.S_final = static_cast<int*>(S_final);
        p.L = L;
        p.C = (int)P.C;
        p.G = (int)P.G;
        p.n_groups = (int)P.n_groups;
        p.n_dvt = P.n_dvt;
        p.dk_g = (int)P.dk;
        p.dv = (int)d_v;
        p.xcd_remap = xcd_ok(grid);
        p.noncausal = !P.causal;
        p.p0_sub = (int)P.sub;
        return hip_status(la::run_chunked_fwd_i8(p, P.DK, P.DVT, P.T, grid, s), "chunked forward launch");
    }
    la::FwdParams p{};
    p.q = static_cast<const unsigned short*>(qm);
    p.k = static_cast<const unsigned short*>(km);
    p.v = static_cast<const unsigned short*>(v);
    p.k_lo = static_cast<const unsigned short*>(klo);
    p.o = o;
    p.P0 = static_cast<const float*>(states);
    p.z0 = static_cast<const float*>(zst);
    p.S_final = static_cast<float*>(S_final);
    p.z_final = static_cast<float*>(z_final);
    p.L = L;
    p.C = (int)P.C;
    p.G = (int)P.G;
    p.n_groups = (int)P.n_groups;
    p.n_dvt = P.n_dvt;
    p.dk_g = (int)P.dk;
    p.dv = (int)d_v;
    p.fmap = fmap_in_kernel;
    p.in_scale = in_scale;
    p.normalize = P.normalize;
    p.out_f32 = out_dt == LA_F32;
    p.xcd_remap = xcd_ok(grid);
    p.noncausal = !P.causal;
    p.out_scale = (scaled_identity && !P.normalize) ? in_scale * in_scale : 1.0f;
    p.state_scale = scaled_identity ? in_scale : 1.0f;
    p.p0_sub = (int)P.sub;
    p.log2_gamma = lg;
    if (lg != 0.0f && !(P.pipe && out_dt == LA_BF16))
        return fail(LA_ERR_UNSUPPORTED, "the decayed recurrence needs the streaming kernel and bf16 output");
    if (P.final_from_scan) {
        p.S_final = nullptr;
        p.z_final = nullptr;
    }
    hipError_t e;
    if (P.pipe && out_dt == LA_BF16) {
        p.k_lo = nullptr;  // its state sums bf16(phi(k)) only
        return hip_status(la::fwd_pipe_bf16(p, P.DK, P.DVT, (int)P.C, grid, s), "chunked forward launch");
    }
    int DVT = P.DVT, T = P.T;
    int64_t grid_g = grid;
    if (P.pipe) {
        // fp32 outputs: the general kernel on the same groups
        DVT = kernel_dvt(d_v);
        T = tile_bf16(P.C, P.DK, DVT, klo != nullptr);
        p.n_dvt = (int)(d_v / DVT);
        grid_g = BH * P.n_groups * p.n_dvt;
        p.xcd_remap = xcd_ok(grid_g);
    }
    switch (P.DK) {
        case 32: e = la::fwd_bf16_dk32(p, DVT, T, grid_g, s); break;
        case 64: e = la::fwd_bf16_dk64(p, DVT, T, grid_g, s); break;
        case 128: e = la::fwd_bf16_dk128(p, DVT, T, grid_g, s); break;
        default: e = la::fwd_bf16_dk256(p, DVT, T, grid_g, s); break;
    }
    return hip_status(e, "chunked forward launch");
}


// ---------------------------------------------------------------------------
// The forward without a workspace argument.  Its scratch is a file-scope device
// array; each device the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in: the device address
// comes from hipGetSymbolAddress, once per device with that device current, and
// only that address is ever passed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

static la_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(LA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress of the scratch array");
        if (ptr == nullptr) return fail(LA_ERR_HIP, "hipGetSymbolAddress gave no address for the scratch array");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return LA_OK;
}


extern "C" {

const char* la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID_ARG: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported";
        case LA_ERR_HIP: return "HIP runtime error";
        case LA_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

const char* la_last_error(void) { return g_last_error; }

int la_version(void) { return 100; }

// ---------------------------------------------------------------------------
la_status la_feature_map(la_fmap f, const void* x, la_dtype xdt, int64_t rows, int64_t d_in, const void* W,
                         int64_t m, float in_scale, void* y, la_dtype ydt, la_stream_t stream) {
    g_last_error[0] = 0;
    if (x == nullptr || y == nullptr) return fail(LA_ERR_INVALID_ARG, "x and y must not be NULL");
    if (rows < 1 || d_in < 1) return fail(LA_ERR_INVALID_ARG, "rows and d_in must be positive");
    if (xdt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "x must be LA_BF16");
    if (ydt != LA_BF16 && ydt != LA_F32) return fail(LA_ERR_UNSUPPORTED, "y must be LA_BF16 or LA_F32");
    if (!(in_scale == in_scale)) return fail(LA_ERR_INVALID_ARG, "in_scale is NaN");
    la::FmapParams p{};
    p.x = static_cast<const unsigned short*>(x);
    p.y = y;
    p.rows = rows;
    p.d_in = (int)d_in;
    p.in_scale = in_scale;
    p.y_f32 = ydt == LA_F32;
    if (f == LA_FMAP_FAVOR) {
        if (W == nullptr) return fail(LA_ERR_INVALID_ARG, "FAVOR+ needs W");
        if (!pow2_in(m, 16, 256)) return fail(LA_ERR_UNSUPPORTED, "m must be 16..256, a power of two");
        if (!pow2_in(d_in, 16, 128)) return fail(LA_ERR_UNSUPPORTED, "d_in must be 16..128, a power of two");
        p.W = static_cast<const unsigned short*>(W);
        p.m = (int)m;
        p.fmap = 2;
    } else if (f == LA_FMAP_ELU1 || f == LA_FMAP_IDENTITY) {
        if (d_in % 8 != 0) return fail(LA_ERR_UNSUPPORTED, "d_in must be a multiple of 8");
        p.fmap = f == LA_FMAP_ELU1 ? 1 : 0;
    } else {
        return fail(LA_ERR_INVALID_ARG, "unknown feature map %d", (int)f);
    }
    return hip_status(la::run_feature_map(p, (hipStream_t)stream), "la_feature_map launch");
}

// ---------------------------------------------------------------------------
static la_status chunk_states_impl(const void* k, const void* v, bool i8, int64_t BH, int64_t L, int64_t d_k,
                                   int64_t d_v, int64_t Cs, int n_items, int n_out, void* S, void* z, int fmap,
                                   float in_scale, hipStream_t s, const void* k_lo = nullptr, float lg = 0.0f) {
    const int DVT = kernel_dvt(d_v);
    const int n_dvt = (int)(d_v / DVT);
    const int64_t grid = BH * (int64_t)n_items * n_dvt;
    if (grid > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
    if (grid == 0) return LA_OK;
    if (i8) {
        la::StatesParamsI8 p{};
        p.k = static_cast<const signed char*>(k);
        p.v = static_cast<const signed char*>(v);
        p.S = static_cast<int*>(S);
        p.z = static_cast<int*>(z);
        p.L = L;
        p.C = Cs;
        p.n_items = n_items;
        p.n_out = n_out;
        p.n_dvt = n_dvt;
        p.dk_g = (int)d_k;
        p.dv = (int)d_v;
        p.xcd_remap = xcd_ok(grid);
        return hip_status(la::run_chunk_states_i8(p, kernel_dk_i8(d_k), DVT, grid, s), "chunk states launch");
    }
    // long runs of whole 64-row tiles at feature width 64, 128 or 256: the
    // streaming kernel (its own value tiling)
    const int dvt_pipe = 64;
    bool stream_ok = (d_k == 64 || d_k == 128 || d_k == 256) && d_v % dvt_pipe == 0 && Cs % 64 == 0 &&
                           Cs >= 256 && (fmap == 0 || fmap == 1) && !(lg != 0.0f && k_lo != nullptr);
    // elu+1 mapped here at feature width 128 or 256 (one streaming workgroup
    // per CU): only when the workgroups fit the CUs in one round; with more,
    // the register-staged kernel at several workgroups per CU hides the
    // mapping better.  At width 64 two streaming workgroups share a CU.
    if (stream_ok && fmap == 1 && k_lo == nullptr && d_k != 64 && BH * (int64_t)n_items * (d_v / dvt_pipe) > 256)
        stream_ok = false;
    la::StatesParams p{};
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.k_lo = static_cast<const unsigned short*>(k_lo);
    p.S = static_cast<float*>(S);
    p.z = static_cast<float*>(z);
    p.L = L;
    p.C = Cs;
    p.n_items = n_items;
    p.n_out = n_out;
    p.n_dvt = n_dvt;
    p.dk_g = (int)d_k;
    p.dv = (int)d_v;
    p.fmap = fmap;
    p.in_scale = in_scale;
    p.want_z = z != nullptr;
    p.xcd_remap = xcd_ok(grid);
    p.log2_gamma = lg;
    if (stream_ok) {
        p.n_dvt = (int)(d_v / dvt_pipe);
        const int64_t sgrid = BH * (int64_t)n_items * p.n_dvt;
        if (sgrid > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
        p.xcd_remap = xcd_ok(sgrid);
        const int kind = k_lo != nullptr ? 2 : (fmap == 1 ? 1 : 0);
        return hip_status(la::states_pipe_bf16(p, (int)d_k, kind, sgrid, s), "chunk states launch");
    }
    hipError_t e;
    switch (kernel_dk_bf16(d_k)) {
        case 32: e = la::states_bf16_dk32(p, DVT, grid, s); break;
        case 64: e = la::states_bf16_dk64(p, DVT, grid, s); break;
        case 128: e = la::states_bf16_dk128(p, DVT, grid, s); break;
        default: e = la::states_bf16_dk256(p, DVT, grid, s); break;
    }
    return hip_status(e, "chunk states launch");
}

static la_status check_gamma(float gamma) {
    if (!(gamma > 0.0f && gamma <= 1.0f)) return fail(LA_ERR_INVALID_ARG, "gamma must lie in (0, 1], got %g", (double)gamma);
    return LA_OK;
}

static float log2_of(float gamma) { return gamma == 1.0f ? 0.0f : (float)std::log2((double)gamma); }

static la_status chunk_states_entry(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                                    int64_t d_k, int64_t d_v, int64_t C, void* S, void* z, float gamma,
                                    la_stream_t stream) {
    if (k == nullptr || v == nullptr || S == nullptr) return fail(LA_ERR_INVALID_ARG, "k, v and S must not be NULL");
    if (BH < 1 || L < 1) return fail(LA_ERR_INVALID_ARG, "BH and L must be positive");
    if (in_dt != LA_BF16 && in_dt != LA_I8) return fail(LA_ERR_UNSUPPORTED, "input type must be LA_BF16 or LA_I8");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k and d_v must be 16..256, powers of two");
    const int64_t Cs = C <= 0 ? 1 : (C > L ? L : C);
    const int64_t N = cdiv(L, Cs);
    if (N > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "too many chunks");
    if (gamma != 1.0f && in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the decayed recurrence needs LA_BF16 inputs");
    return chunk_states_impl(k, v, in_dt == LA_I8, BH, L, d_k, d_v, Cs, (int)N, (int)N, S, z, la::FMAP_NONE, 1.0f,
                             (hipStream_t)stream, nullptr, log2_of(gamma));
}

la_status la_chunk_states(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k,
                          int64_t d_v, int64_t C, void* S, void* z, la_stream_t stream) {
    g_last_error[0] = 0;
    return chunk_states_entry(k, v, in_dt, BH, L, d_k, d_v, C, S, z, 1.0f, stream);
}

la_status la_chunk_states_decay(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k,
                                int64_t d_v, int64_t C, float gamma, void* S, void* z, la_stream_t stream) {
    g_last_error[0] = 0;
    const la_status st = check_gamma(gamma);
    if (st != LA_OK) return st;
    return chunk_states_entry(k, v, in_dt, BH, L, d_k, d_v, C, S, z, gamma, stream);
}

// ---------------------------------------------------------------------------
static la_status state_scan_entry(void* S, void* z, la_dtype st_dt, int64_t BH, int64_t N, int64_t d_k,
                                  int64_t d_v, int64_t L, int64_t C, float gamma, void* S_final, void* z_final,
                                  la_stream_t stream) {
    if (S == nullptr) return fail(LA_ERR_INVALID_ARG, "S must not be NULL");
    if (BH < 1 || N < 1) return fail(LA_ERR_INVALID_ARG, "BH and N must be positive");
    if (st_dt != LA_F32 && st_dt != LA_I32) return fail(LA_ERR_UNSUPPORTED, "state type must be LA_F32 or LA_I32");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k and d_v must be 16..256, powers of two");
    if (z == nullptr && z_final != nullptr) return fail(LA_ERR_INVALID_ARG, "z_final needs z");
    la::ScanParams p{};
    p.S = S;
    p.z = z;
    p.S_final = S_final;
    p.z_final = z_final;
    p.N = N;
    p.E = d_k * d_v;
    p.Ez = d_k;
    p.is_int = st_dt == LA_I32;
    if (gamma != 1.0f) {
        if (st_dt != LA_F32) return fail(LA_ERR_UNSUPPORTED, "the decayed prefix needs LA_F32 states");
        if (L < 1) return fail(LA_ERR_INVALID_ARG, "L must be positive");
        const int64_t Cs = C <= 0 ? 1 : (C > L ? L : C);
        if (cdiv(L, Cs) != N) return fail(LA_ERR_INVALID_ARG, "N must be ceil(L / C)");
        p.log2_gamma = log2_of(gamma);
        p.L = L;
        p.Cs = Cs;
    }
    return hip_status(la::run_state_scan(p, BH, (hipStream_t)stream), "state scan launch");
}

la_status la_state_scan(void* S, void* z, la_dtype st_dt, int64_t BH, int64_t N, int64_t d_k, int64_t d_v,
                        void* S_final, void* z_final, la_stream_t stream) {
    g_last_error[0] = 0;
    return state_scan_entry(S, z, st_dt, BH, N, d_k, d_v, 0, 0, 1.0f, S_final, z_final, stream);
}

la_status la_state_scan_decay(void* S, void* z, la_dtype st_dt, int64_t BH, int64_t N, int64_t d_k, int64_t d_v,
                              int64_t L, int64_t C, float gamma, void* S_final, void* z_final, la_stream_t stream) {
    g_last_error[0] = 0;
    const la_status st = check_gamma(gamma);
    if (st != LA_OK) return st;
    return state_scan_entry(S, z, st_dt, BH, N, d_k, d_v, L, C, gamma, S_final, z_final, stream);
}

// ---------------------------------------------------------------------------
size_t la_chunked_forward_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                                    int causal, int normalize, la_fmap f, int64_t m, float in_scale,
                                    int64_t group) {
    Plan P{};
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    // the decayed forward takes the same workspace: the larger of the two plans
    la_status s = make_plan(P, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, in_scale, group, false);
    size_t ws = P.ws_total;
    if (s == LA_OK) {
        Plan Pd{};
        if (make_plan(Pd, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, in_scale, group, true) == LA_OK)
            ws = std::max(ws, Pd.ws_total);
        // and the plan of a bf16 output (FAVOR+ mapped in the kernels)
        Plan Pb{};
        if (make_plan(Pb, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, in_scale, group, false, true) == LA_OK)
            ws = std::max(ws, Pb.ws_total);
    }
    memcpy(g_last_error, saved, sizeof(saved));
    if (s != LA_OK) return 0;
    return ws;
}

int64_t la_chunked_forward_group(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_in, int64_t d_v, int64_t C,
                                 int causal, int normalize, la_fmap f, int64_t m, int64_t group) {
    Plan P{};
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    const la_status s = make_plan(P, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, 1.0f, group, false,
                                  in_dt == LA_BF16);
    memcpy(g_last_error, saved, sizeof(saved));
    return s == LA_OK ? P.G : 0;
}

// FAVOR+ mapped inside the kernels: phase 1 sums each run's phi(k)^T v (and
// phi(k)) from the raw keys, the scan forms the groups' prefixes and the total,
// and phase 3 maps q and k of each chunk as it streams the group.
static la_status favor_forward(const Plan& P, const void* q, const void* k, const void* v, const void* W,
                               float in_scale, void* o, void* S_final, void* z_final, char* ws, hipStream_t s) {
    const int64_t BH = P.BH;
    float* states = P.ws_states ? reinterpret_cast<float*>(ws) : nullptr;
    float* zst = P.ws_z ? reinterpret_cast<float*>(ws + P.ws_states) : nullptr;
    la::FavorParams fp{};
    fp.q = static_cast<const unsigned short*>(q);
    fp.k = static_cast<const unsigned short*>(k);
    fp.v = static_cast<const unsigned short*>(v);
    fp.W = static_cast<const unsigned short*>(W);
    fp.L = P.L;
    fp.dv = (int)P.dv;
    fp.n_dvt = P.n_dvt;
    fp.in_scale = in_scale;
    const bool want_final = S_final != nullptr || z_final != nullptr;
    if (P.n_groups > 1 || want_final) {
        const int64_t n_slots = P.n_groups * P.sub;
        const int64_t n_items = want_final ? n_slots : n_slots - P.sub;
        const int64_t rows = P.G * P.C / P.sub;  // a multiple of 64 (planned so)
        if (rows % 64 != 0 || states == nullptr || (P.normalize && zst == nullptr))
            return fail(LA_ERR_UNSUPPORTED, "FAVOR+ phase-1 plan: rows %lld", (long long)rows);
        fp.S = states;
        fp.z = zst;
        fp.rows = rows;
        fp.n_groups = (int)n_items;
        fp.n_out = (int)n_slots;
        const int64_t grid1 = BH * n_items * P.n_dvt;
        fp.xcd_remap = xcd_ok(grid1);
        la_status st = hip_status(la::run_favor_states(fp, (int)P.dk, P.normalize, grid1, s), "FAVOR+ states launch");
        if (st != LA_OK) return st;
        la::ScanParams sp{};
        sp.S = states;
        sp.z = zst;
        sp.N = n_slots;
        sp.L = P.L;
        sp.Cs = rows;
        if (want_final) {
            sp.S_final = S_final;
            sp.z_final = z_final;
        }
        sp.E = P.dk * P.dv;
        sp.Ez = P.dk;
        st = hip_status(la::run_state_scan(sp, BH, s), "state scan launch");
        if (st != LA_OK) return st;
    }
    fp.S = nullptr;
    fp.z = nullptr;
    fp.rows = 0;
    fp.n_out = 0;
    fp.o = static_cast<unsigned short*>(o);
    fp.P0 = P.n_groups > 1 ? states : nullptr;
    fp.z0 = P.n_groups > 1 ? zst : nullptr;
    fp.G = (int)P.G;
    fp.n_groups = (int)P.n_groups;
    fp.p0_sub = (int)P.sub;
    const int64_t grid = BH * P.n_groups * P.n_dvt;
    fp.xcd_remap = xcd_ok(grid);
    return hip_status(la::run_favor_fwd(fp, (int)P.dk, P.normalize, grid, s), "FAVOR+ forward launch");
}

static la_status forward_entry(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                               int64_t d_in, int64_t d_v, int64_t C, int causal, int normalize, la_fmap f,
                               const void* W, int64_t m, float in_scale, float gamma, void* o, la_dtype out_dt,
                               void* S_final, void* z_final, int64_t group, void* workspace, size_t ws_bytes,
                               la_stream_t stream) {
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    la_status st = check_dtypes_forward(in_dt, out_dt, normalize, f, in_scale);
    if (st != LA_OK) return st;
    if (f == LA_FMAP_FAVOR && W == nullptr) return fail(LA_ERR_INVALID_ARG, "FAVOR+ needs W");
    if (z_final != nullptr && !normalize) return fail(LA_ERR_INVALID_ARG, "z_final needs normalize");
    Plan P{};
    const float lg = log2_of(gamma);
    st = make_plan(P, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, in_scale, group, lg != 0.0f,
                   out_dt == LA_BF16);
    if (st != LA_OK) return st;
    if (lg != 0.0f && !(causal && P.pipe && out_dt == LA_BF16))
        return fail(LA_ERR_UNSUPPORTED,
                    "the decayed recurrence runs on the streaming kernel: causal, bf16 in and out, C in {32, 64, 128} "
                    "with d_k in {64, 128} and d_v a multiple of 64, or C in {32, 64} with d_k = 256");
    if (P.ws_total > 0 && (workspace == nullptr || ws_bytes < P.ws_total))
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", P.ws_total,
                    workspace ? ws_bytes : (size_t)0);
    hipStream_t s = (hipStream_t)stream;
    char* ws = static_cast<char*>(workspace);
    if (P.favor) return favor_forward(P, q, k, v, W, in_scale, o, S_final, z_final, ws, s);
    const void* qm = q;
    const void* km = k;
    const void* klo = nullptr;
    int fmap_in_kernel = la::FMAP_NONE;
    if (P.premap) {
        void* qp = ws;
        void* kp = ws + P.ws_phi;
        void* kl = ws + 2 * P.ws_phi;
        la_status a = la_feature_map(f, q, LA_BF16, BH * L, d_in, W, m, in_scale, qp, LA_BF16, stream);
        if (a != LA_OK) return a;
        la::FmapParams fp{};
        fp.x = static_cast<const unsigned short*>(k);
        fp.W = static_cast<const unsigned short*>(W);
        fp.y = kp;
        fp.y_lo = static_cast<unsigned short*>(kl);
        fp.rows = BH * L;
        fp.d_in = (int)d_in;
        fp.m = f == LA_FMAP_FAVOR ? (int)m : (int)d_in;
        fp.fmap = f == LA_FMAP_FAVOR ? 2 : 1;
        fp.in_scale = in_scale;
        a = hip_status(la::run_feature_map(fp, s), "feature map launch");
        if (a != LA_OK) return a;
        qm = qp;
        km = kp;
        klo = kl;
        ws += 3 * P.ws_phi;
    } else if (f == LA_FMAP_ELU1) {
        fmap_in_kernel = la::FMAP_ELU1;
    }
    void* states = P.ws_states ? ws : nullptr;
    void* zst = P.ws_z ? ws + P.ws_states : nullptr;

    // phase 1 + 2 at group granularity (or the total state for non-causal);
    // with the final state from the scan, phase 1 also sums the last group
    const bool want_final = P.final_from_scan && (S_final != nullptr || z_final != nullptr);
    if (P.causal && (P.n_groups > 1 || want_final)) {
        const int64_t n_slots = P.n_groups * P.sub;
        const int64_t n_items = want_final ? n_slots : n_slots - P.sub;
        const int64_t Cs = P.G * P.C / P.sub;
        st = chunk_states_impl(km, v, P.i8, BH, L, P.dk, d_v, Cs, (int)n_items, (int)n_slots, states, zst,
                               fmap_in_kernel, in_scale, s, klo, lg);
        if (st != LA_OK) return st;
        la::ScanParams sp{};
        sp.S = states;
        sp.z = zst;
        sp.N = n_slots;
        sp.log2_gamma = lg;
        sp.L = L;
        sp.Cs = Cs;
        if (want_final) {
            sp.S_final = S_final;
            sp.z_final = z_final;
        }
        sp.E = P.dk * d_v;
        sp.Ez = P.dk;
        sp.is_int = P.i8;
        st = hip_status(la::run_state_scan(sp, BH, s), "state scan launch");
        if (st != LA_OK) return st;
    } else if (!P.causal) {
        st = chunk_states_impl(km, v, P.i8, BH, L, P.dk, d_v, L, 1, 1, states, zst, fmap_in_kernel, in_scale, s, klo);
        if (st != LA_OK) return st;
    }

    // phase 3
    return launch_phase3(P, qm, km, klo, v, o, out_dt, states, zst, S_final, z_final, fmap_in_kernel, in_scale,
                         f == LA_FMAP_IDENTITY && in_scale != 1.0f, s, lg);
}

la_status la_chunked_forward(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                             int64_t d_in, int64_t d_v, int64_t C, int causal, int normalize, la_fmap f,
                             const void* W, int64_t m, float in_scale, void* o, la_dtype out_dt, void* S_final,
                             void* z_final, int64_t group, void* workspace, size_t ws_bytes,
                             la_stream_t stream) {
    g_last_error[0] = 0;
    return forward_entry(q, k, v, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, W, m, in_scale, 1.0f, o, out_dt,
                         S_final, z_final, group, workspace, ws_bytes, stream);
}

la_status la_chunked_forward_noalloc(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                     int64_t L, int64_t d_in, int64_t d_v, int64_t C, int causal, int normalize,
                                     la_fmap f, const void* W, int64_t m, float in_scale, void* o, la_dtype out_dt,
                                     void* S_final, void* z_final, int64_t group, la_stream_t stream) {
    g_last_error[0] = 0;
    Plan P{};
    la_status st = make_plan(P, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, m, in_scale, group, false,
                             out_dt == LA_BF16);
    if (st != LA_OK) return st;
    if (P.ws_total > (size_t)LA_NOALLOC_SCRATCH_BYTES)
        return fail(LA_ERR_UNSUPPORTED,
                    "this forward needs %zu bytes of scratch; the allocation-free forward holds at most %zu "
                    "(la_chunked_forward takes a workspace of any size)",
                    P.ws_total, (size_t)LA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (P.ws_total > 0) {
        st = scratch_of_current_device(&ws);
        if (st != LA_OK) return st;
    }
    return forward_entry(q, k, v, in_dt, BH, L, d_in, d_v, C, causal, normalize, f, W, m, in_scale, 1.0f, o, out_dt,
                         S_final, z_final, group, ws, ws ? (size_t)LA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

la_status la_chunked_forward_decay(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                   int64_t L, int64_t d_in, int64_t d_v, int64_t C, int normalize, la_fmap f,
                                   const void* W, int64_t m, float in_scale, float gamma, void* o, la_dtype out_dt,
                                   void* S_final, void* z_final, int64_t group, void* workspace, size_t ws_bytes,
                                   la_stream_t stream) {
    g_last_error[0] = 0;
    const la_status st = check_gamma(gamma);
    if (st != LA_OK) return st;
    return forward_entry(q, k, v, in_dt, BH, L, d_in, d_v, C, 1, normalize, f, W, m, in_scale, gamma, o, out_dt,
                         S_final, z_final, group, workspace, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
static la_status chunk_output_entry(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                    int64_t L, int64_t d_k, int64_t d_v, int64_t C, int64_t group,
                                    const void* P_prefix, const void* z_prefix, int normalize, float gamma, void* o,
                                    la_dtype out_dt, void* S_final, void* z_final, la_stream_t stream) {
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    la_status st = check_dtypes_forward(in_dt, out_dt, normalize, LA_FMAP_IDENTITY, 1.0f);
    if (st != LA_OK) return st;
    if (z_final != nullptr && !normalize) return fail(LA_ERR_INVALID_ARG, "z_final needs normalize");
    if (group < 1) return fail(LA_ERR_INVALID_ARG, "group must be at least 1");
    Plan P{};
    // planned without the decay, which may round the group: the caller's
    // prefixes are laid out at exactly this group size
    st = make_plan(P, in_dt, BH, L, d_k, d_v, C, 1, normalize, LA_FMAP_IDENTITY, 0, 1.0f, group, false);
    if (st != LA_OK) return st;
    if (P.G != (group < P.n_chunks ? group : P.n_chunks))
        return fail(LA_ERR_UNSUPPORTED, "group %lld cannot be kept for these arguments", (long long)group);
    if (P.n_groups > 1 && (P_prefix == nullptr || (normalize && z_prefix == nullptr)))
        return fail(LA_ERR_INVALID_ARG, "more than one group needs the prefix states (and normalisers)");
    P.sub = 1;  // the caller's prefixes: one per group
    const float lg = log2_of(gamma);
    if (lg != 0.0f && !(P.pipe && out_dt == LA_BF16))
        return fail(LA_ERR_UNSUPPORTED,
                    "the decayed recurrence runs on the streaming kernel: bf16 in and out, C in {32, 64, 128} with d_k "
                    "in {64, 128} and d_v a multiple of 64, or C in {32, 64} with d_k = 256; at C = 32 an even group");
    return launch_phase3(P, q, k, nullptr, v, o, out_dt, P_prefix, z_prefix, S_final, z_final, la::FMAP_NONE,
                         1.0f, false, (hipStream_t)stream, lg);
}

la_status la_chunk_output(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                          int64_t d_k, int64_t d_v, int64_t C, int64_t group, const void* P_prefix,
                          const void* z_prefix, int normalize, void* o, la_dtype out_dt, void* S_final,
                          void* z_final, la_stream_t stream) {
    g_last_error[0] = 0;
    return chunk_output_entry(q, k, v, in_dt, BH, L, d_k, d_v, C, group, P_prefix, z_prefix, normalize, 1.0f, o,
                              out_dt, S_final, z_final, stream);
}

la_status la_chunk_output_decay(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                int64_t L, int64_t d_k, int64_t d_v, int64_t C, int64_t group, const void* P_prefix,
                                const void* z_prefix, int normalize, float gamma, void* o, la_dtype out_dt,
                                void* S_final, void* z_final, la_stream_t stream) {
    g_last_error[0] = 0;
    const la_status st = check_gamma(gamma);
    if (st != LA_OK) return st;
    return chunk_output_entry(q, k, v, in_dt, BH, L, d_k, d_v, C, group, P_prefix, z_prefix, normalize, gamma, o,
                              out_dt, S_final, z_final, stream);
}

// ---------------------------------------------------------------------------
// Log-linear attention (chunks of 64): per-chunk states, their bucket
// pyramid, then the output kernel.
static int64_t loglinear_levels_of(int64_t L) {
    int64_t b = 0;
    for (int64_t x = L - 1; x > 0; x >>= 1) ++b;
    return 1 + b;
}

static int64_t loglinear_pyramid_nodes(int64_t N) {
    int64_t total = 0;
    for (int64_t nodes = N; nodes >= 2;) {
        nodes /= 2;
        total += nodes;
    }
    return total;
}

static la_status loglinear_check(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v, int64_t C,
                                 size_t* ws_S, size_t* ws_T) {
    if (BH < 1 || L < 1) return fail(LA_ERR_INVALID_ARG, "BH and L must be positive");
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "log-linear attention takes LA_BF16 inputs");
    if (C != 64) return fail(LA_ERR_UNSUPPORTED, "log-linear attention runs on chunks of 64 rows");
    if (d_k != 64 && d_k != 128) return fail(LA_ERR_UNSUPPORTED, "log-linear attention needs d_k of 64 or 128");
    if (!pow2_in(d_v, 64, 256)) return fail(LA_ERR_UNSUPPORTED, "log-linear attention needs d_v of 64, 128 or 256");
    if (loglinear_levels_of(L) > 40) return fail(LA_ERR_UNSUPPORTED, "sequence too long");
    const int64_t N = cdiv(L, C);
    if (BH * N * (d_v / 64) > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
    *ws_S = N > 1 ? align256((size_t)(BH * N * d_k * d_v * 4)) : 0;
    *ws_T = align256((size_t)(BH * loglinear_pyramid_nodes(N) * d_k * d_v * 2));  // bf16 nodes
    return LA_OK;
}

int64_t la_loglinear_levels(int64_t L) { return L < 1 ? 0 : loglinear_levels_of(L); }

static la_status loglinear_prefix_check(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v,
                                        size_t* ws) {
    if (BH < 1 || L < 1 || d_k < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the log-linear prefix levels take LA_BF16 inputs");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k=%lld, d_v=%lld: powers of two in 16..256", (long long)d_k,
                    (long long)d_v);
    if (loglinear_levels_of(L) > 40) return fail(LA_ERR_UNSUPPORTED, "sequence too long");
    // the states of the whole chunks of 64 rows before the last row's chunk
    *ws = align256((size_t)BH * (size_t)((L - 1) >> 6) * (size_t)(d_k * d_v) * 4);
    return LA_OK;
}

size_t la_loglinear_prefix_levels_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v) {
    size_t ws = 0;
    if (loglinear_prefix_check(in_dt, BH, L, d_k, d_v, &ws) != LA_OK) return 0;
    return ws;
}

la_status la_loglinear_prefix_levels(const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                                     int64_t d_k, int64_t d_v, int64_t n_levels, float* S, void* workspace,
                                     size_t ws_bytes, la_stream_t stream) {
    g_last_error[0] = 0;
    if (k == nullptr || v == nullptr || S == nullptr) return fail(LA_ERR_INVALID_ARG, "k, v and S must not be NULL");
    size_t ws = 0;
    la_status st = loglinear_prefix_check(in_dt, BH, L, d_k, d_v, &ws);
    if (st != LA_OK) return st;
    if (n_levels < loglinear_levels_of(L) || n_levels > 40)
        return fail(LA_ERR_INVALID_ARG, "n_levels=%lld: %lld tokens need %lld..40", (long long)n_levels,
                    (long long)L, (long long)loglinear_levels_of(L));
    if (ws > 0 && (workspace == nullptr || ws_bytes < ws))
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws, workspace ? ws_bytes : (size_t)0);
    hipStream_t s = (hipStream_t)stream;
    const int64_t n_chunks = (L - 1) >> 6;
    if (n_chunks > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "too many chunks");
    if (n_chunks > 0) {
        st = chunk_states_impl(k, v, false, BH, L, d_k, d_v, 64, (int)n_chunks, (int)n_chunks, workspace, nullptr,
                               0, 1.0f, s);
        if (st != LA_OK) return st;
    }
    la::LogLinPrefixParams p{};
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.chunks = n_chunks > 0 ? static_cast<const float*>(workspace) : nullptr;
    p.S = S;
    p.BH = BH;
    p.L = L;
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    p.n_lev = (int)n_levels;
    p.n_chunks = (int)n_chunks;
    return hip_status(la::run_loglinear_prefix_levels(p, s), "log-linear prefix levels launch");
}

la_status la_recurrent_step_loglinear(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                                      int64_t d_k, int64_t d_v, const float* lam, int64_t n_levels, int64_t t,
                                      float* S, void* o, la_dtype out_dt, la_stream_t stream) {
    g_last_error[0] = 0;
    if (q == nullptr || k == nullptr || v == nullptr || lam == nullptr || S == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, lam, S and o must not be NULL");
    if (n_states < 1 || d_k < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (t < 0) return fail(LA_ERR_INVALID_ARG, "position t=%lld is negative", (long long)t);
    int64_t need = 1;  // 1 + the bit length of t
    for (int64_t x = t; x > 0; x >>= 1) ++need;
    if (n_levels < need || n_levels > 40)
        return fail(LA_ERR_INVALID_ARG, "n_levels=%lld: position %lld needs %lld..40", (long long)n_levels,
                    (long long)t, (long long)need);
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the log-linear step takes LA_BF16 inputs");
    if (out_dt != LA_F32 && out_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "output must be LA_F32 or LA_BF16");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k=%lld, d_v=%lld: powers of two in 16..256", (long long)d_k,
                    (long long)d_v);
    if (n_states > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "too many states");
    la::LogLinStepParams p{};
    p.q = static_cast<const unsigned short*>(q);
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.lam = lam;
    p.S = S;
    p.o = o;
    p.n = n_states;
    p.t = t;
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    p.n_lev = (int)n_levels;
    p.out_f32 = out_dt == LA_F32;
    return hip_status(la::run_loglinear_step(p, (hipStream_t)stream), "log-linear step launch");
}

size_t la_loglinear_forward_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v, int64_t C) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    size_t a = 0, b = 0;
    const la_status st = loglinear_check(in_dt, BH, L, d_k, d_v, C, &a, &b);
    memcpy(g_last_error, saved, sizeof(saved));
    return st == LA_OK ? a + b : 0;
}

la_status la_loglinear_forward(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH, int64_t L,
                               int64_t d_k, int64_t d_v, int64_t C, const float* lam, int64_t n_levels, void* o,
                               la_dtype out_dt, float* S_levels, int64_t n_state_levels, void* workspace,
                               size_t ws_bytes, la_stream_t stream) {
    g_last_error[0] = 0;
    if (q == nullptr || k == nullptr || v == nullptr || lam == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, lam and o must not be NULL");
    size_t ws_S = 0, ws_T = 0;
    la_status st = loglinear_check(in_dt, BH, L, d_k, d_v, C, &ws_S, &ws_T);
    if (st != LA_OK) return st;
    if (out_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "log-linear attention writes LA_BF16 outputs");
    if (n_levels != loglinear_levels_of(L))
        return fail(LA_ERR_INVALID_ARG, "lam must hold %lld levels per token for L = %lld, got %lld",
                    (long long)loglinear_levels_of(L), (long long)L, (long long)n_levels);
    if (S_levels != nullptr && (n_state_levels < n_levels || n_state_levels > 40))
        return fail(LA_ERR_INVALID_ARG, "n_state_levels=%lld: %lld tokens need %lld..40", (long long)n_state_levels,
                    (long long)L, (long long)n_levels);
    if (ws_S + ws_T > 0 && (workspace == nullptr || ws_bytes < ws_S + ws_T))
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws_S + ws_T,
                    workspace ? ws_bytes : (size_t)0);
    hipStream_t s = (hipStream_t)stream;
    const int64_t N = cdiv(L, C);
    char* ws = static_cast<char*>(workspace);
    float* S = N > 1 ? reinterpret_cast<float*>(ws) : nullptr;
    unsigned short* T = ws_T > 0 ? reinterpret_cast<unsigned short*>(ws + ws_S) : nullptr;
    if (N > 1) {
        st = chunk_states_impl(k, v, false, BH, L, d_k, d_v, C, (int)N, (int)N, S, nullptr, la::FMAP_NONE, 1.0f, s);
        if (st != LA_OK) return st;
        st = hip_status(la::run_loglinear_pyramid(S, T, BH, (int)N, (int)loglinear_pyramid_nodes(N), d_k * d_v,
                                                  S_levels, L - 1, (int)n_state_levels, s),
                        "log-linear pyramid launch");
        if (st != LA_OK) return st;
    }
    la::LogLinParams p{};
    p.q = static_cast<const unsigned short*>(q);
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.lam = lam;
    p.S = S;
    p.T = T;
    p.o = static_cast<unsigned short*>(o);
    p.L = L;
    p.N = (int)N;
    p.n_pyr = (int)loglinear_pyramid_nodes(N);
    p.n_lev = (int)n_levels;
    p.n_dvt = (int)(d_v / 64);
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    const int64_t grid = BH * N * p.n_dvt;
    p.xcd_remap = xcd_ok(grid);
    st = hip_status(la::run_loglinear_fwd(p, grid, s), "log-linear forward launch");
    if (st != LA_OK || S_levels == nullptr) return st;
    // the level states after the last token: levels of two chunks or more were
    // written by the pyramid above; level 7 is one chunk state, the rest rows
    la::LogLinPrefixParams lp{};
    lp.k = p.k;
    lp.v = p.v;
    lp.chunks = S;
    lp.S = S_levels;
    lp.BH = BH;
    lp.L = L;
    lp.dk = (int)d_k;
    lp.dv = (int)d_v;
    lp.n_lev = (int)n_state_levels;
    lp.n_chunks = N > 1 ? (int)N : 0;
    lp.pyr_written = N > 1 ? 1 : 0;
    return hip_status(la::run_loglinear_prefix_levels(lp, s), "log-linear level states launch");
}

// ---------------------------------------------------------------------------
static la_status step_entry(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                            int64_t d_in, int64_t d_v, la_fmap f, const void* W, int64_t m, float in_scale,
                            int normalize, float gamma, float* S, float* z, void* o, la_dtype out_dt,
                            la_stream_t stream) {
    if (q == nullptr || k == nullptr || v == nullptr || S == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, S and o must not be NULL");
    if (normalize && z == nullptr) return fail(LA_ERR_INVALID_ARG, "normalize needs z");
    if (n_states < 1 || d_in < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "decode inputs must be LA_BF16");
    if (out_dt != LA_F32 && out_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "decode output must be LA_F32 or LA_BF16");
    if (!(in_scale == in_scale)) return fail(LA_ERR_INVALID_ARG, "in_scale is NaN");
    int64_t dk = d_in;
    int fm = 0;
    if (f == LA_FMAP_FAVOR) {
        if (W == nullptr) return fail(LA_ERR_INVALID_ARG, "FAVOR+ needs W");
        if (!pow2_in(m, 16, 256) || !pow2_in(d_in, 16, 128))
            return fail(LA_ERR_UNSUPPORTED, "FAVOR+ needs m in 16..256 and d_in in 16..128 (powers of two)");
        dk = m;
        fm = 2;
    } else if (f == LA_FMAP_ELU1) {
        fm = 1;
    } else if (f != LA_FMAP_IDENTITY) {
        return fail(LA_ERR_INVALID_ARG, "unknown feature map %d", (int)f);
    }
    if (!pow2_in(dk, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k and d_v must be 16..256, powers of two");
    la::DecodeParams p{};
    p.q = static_cast<const unsigned short*>(q);
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.W = static_cast<const unsigned short*>(W);
    p.S = S;
    p.z = z;
    p.o = o;
    p.n = n_states;
    p.d_in = (int)d_in;
    p.dk = (int)dk;
    p.dv = (int)d_v;
    p.fmap = fm;
    p.in_scale = in_scale;
    p.normalize = normalize != 0;
    p.out_f32 = out_dt == LA_F32;
    p.gamma = gamma;
    return hip_status(la::run_recurrent_step(p, (hipStream_t)stream), "recurrent step launch");
}

la_status la_recurrent_step(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                            int64_t d_in, int64_t d_v, la_fmap f, const void* W, int64_t m, float in_scale,
                            int normalize, float* S, float* z, void* o, la_dtype out_dt, la_stream_t stream) {
    g_last_error[0] = 0;
    return step_entry(q, k, v, in_dt, n_states, d_in, d_v, f, W, m, in_scale, normalize, 1.0f, S, z, o, out_dt,
                      stream);
}

la_status la_recurrent_step_i8(const void* q, const void* k, const void* v, int64_t n_states, int64_t d_k,
                               int64_t d_v, int32_t* S, int32_t* o, la_stream_t stream) {
    g_last_error[0] = 0;
    if (q == nullptr || k == nullptr || v == nullptr || S == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, S and o must not be NULL");
    if (n_states < 1 || d_k < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k=%lld, d_v=%lld: powers of two in 16..256", (long long)d_k,
                    (long long)d_v);
    if (n_states > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "too many states");
    if ((reinterpret_cast<uintptr_t>(S) & 15) != 0) return fail(LA_ERR_INVALID_ARG, "S must be 16-byte aligned");
    la::DecodeParamsI8 p{};
    p.q = static_cast<const signed char*>(q);
    p.k = static_cast<const signed char*>(k);
    p.v = static_cast<const signed char*>(v);
    p.S = S;
    p.o = o;
    p.n = n_states;
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    return hip_status(la::run_recurrent_step_i8(p, (hipStream_t)stream), "int8 step launch");
}

la_status la_recurrent_step_decay(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                                  int64_t d_in, int64_t d_v, la_fmap f, const void* W, int64_t m, float in_scale,
                                  int normalize, float gamma, float* S, float* z, void* o, la_dtype out_dt,
                                  la_stream_t stream) {
    g_last_error[0] = 0;
    const la_status st = check_gamma(gamma);
    if (st != LA_OK) return st;
    return step_entry(q, k, v, in_dt, n_states, d_in, d_v, f, W, m, in_scale, normalize, gamma, S, z, o, out_dt,
                      stream);
}

// ---------------------------------------------------------------------------
// the delta rule
// ---------------------------------------------------------------------------
static constexpr int64_t kDeltaChunk = 64;

static la_status delta_sizes(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v, int64_t C) {
    if (BH < 1 || L < 1 || d_k < 1 || d_v < 1) return fail(LA_ERR_INVALID_ARG, "sizes must be positive");
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the delta rule takes LA_BF16 inputs");
    if (C != kDeltaChunk) return fail(LA_ERR_UNSUPPORTED, "the delta-rule forward runs chunks of 64 rows (C = 64)");
    if (d_k != 64 && d_k != 128) return fail(LA_ERR_UNSUPPORTED, "the delta-rule forward needs d_k in {64, 128}");
    if (d_v % 64 != 0 || !pow2_in(d_v, 64, 256)) return fail(LA_ERR_UNSUPPORTED, "the delta-rule forward needs d_v in {64, 128, 256}");
    if (BH * L > ((int64_t)1 << 40) || BH * (d_v / 64) > 0x7FFFFFFFLL || BH * cdiv(L, kDeltaChunk) > 0x7FFFFFFFLL)
        return fail(LA_ERR_UNSUPPORTED, "problem too large");
    return LA_OK;
}

static size_t delta_ws_T(int64_t BH, int64_t N) { return align256((size_t)BH * N * kDeltaChunk * kDeltaChunk * 2); }
static size_t delta_ws_lg(int64_t BH, int64_t N) { return align256((size_t)BH * N * kDeltaChunk * 4); }

size_t la_chunked_forward_delta_workspace(la_dtype in_dt, int64_t BH, int64_t L, int64_t d_k, int64_t d_v,
                                          int64_t C) {
    char saved[sizeof(g_last_error)];
    memcpy(saved, g_last_error, sizeof(saved));
    const la_status st = delta_sizes(in_dt, BH, L, d_k, d_v, C);
    memcpy(g_last_error, saved, sizeof(saved));
    if (st != LA_OK) return 0;
    const int64_t N = cdiv(L, kDeltaChunk);
    return delta_ws_T(BH, N) + delta_ws_lg(BH, N);
}

la_status la_delta_chunk_transform(const void* k, const float* beta, const float* alpha, la_dtype in_dt,
                                   int64_t BH, int64_t L, int64_t d_k, int64_t C, void* T, float* lg,
                                   la_stream_t stream) {
    g_last_error[0] = 0;
    if (k == nullptr || beta == nullptr || T == nullptr || lg == nullptr)
        return fail(LA_ERR_INVALID_ARG, "k, beta, T and lg must not be NULL");
    la_status st = delta_sizes(in_dt, BH, L, d_k, 64, C);
    if (st != LA_OK) return st;
    la::DeltaPrepParams p{};
    p.k = static_cast<const unsigned short*>(k);
    p.beta = beta;
    p.alpha = alpha;
    p.T = static_cast<unsigned short*>(T);
    p.lg = lg;
    p.BH = BH;
    p.L = L;
    p.N = cdiv(L, kDeltaChunk);
    p.dk = (int)d_k;
    return hip_status(la::run_delta_transform(p, (hipStream_t)stream), "delta transform launch");
}

la_status la_chunked_forward_delta(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t BH,
                                   int64_t L, int64_t d_k, int64_t d_v, int64_t C, const float* beta,
                                   const float* alpha, void* o, la_dtype out_dt, float* S_final, void* workspace,
                                   size_t ws_bytes, la_stream_t stream) {
    g_last_error[0] = 0;
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, beta and o must not be NULL");
    la_status st = delta_sizes(in_dt, BH, L, d_k, d_v, C);
    if (st != LA_OK) return st;
    if (out_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the delta-rule forward writes LA_BF16 outputs");
    const int64_t N = cdiv(L, kDeltaChunk);
    const size_t need = delta_ws_T(BH, N) + delta_ws_lg(BH, N);
    if (workspace == nullptr || ws_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
    char* ws = static_cast<char*>(workspace);
    unsigned short* T = reinterpret_cast<unsigned short*>(ws);
    float* lg = reinterpret_cast<float*>(ws + delta_ws_T(BH, N));
    st = la_delta_chunk_transform(k, beta, alpha, in_dt, BH, L, d_k, C, T, lg, stream);
    if (st != LA_OK) return st;
    la::DeltaFwdParams p{};
    p.q = static_cast<const unsigned short*>(q);
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.T = T;
    p.lg = lg;
    p.o = static_cast<unsigned short*>(o);
    p.S_final = S_final;
    p.BH = BH;
    p.L = L;
    p.N = N;
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    p.n_dvt = (int)(d_v / 64);
    p.xcd_remap = xcd_ok(BH * p.n_dvt);
    return hip_status(la::run_delta_fwd(p, (hipStream_t)stream), "delta forward launch");
}

la_status la_recurrent_step_delta(const void* q, const void* k, const void* v, la_dtype in_dt, int64_t n_states,
                                  int64_t d_k, int64_t d_v, const float* beta, const float* alpha, float* S,
                                  void* o, la_dtype out_dt, la_stream_t stream) {
    g_last_error[0] = 0;
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || S == nullptr || o == nullptr)
        return fail(LA_ERR_INVALID_ARG, "q, k, v, beta, S and o must not be NULL");
    if (n_states < 1) return fail(LA_ERR_INVALID_ARG, "n_states must be positive");
    if (n_states > 0x7FFFFFFFLL) return fail(LA_ERR_UNSUPPORTED, "too many states");
    if (in_dt != LA_BF16) return fail(LA_ERR_UNSUPPORTED, "the delta rule takes LA_BF16 inputs");
    if (out_dt != LA_BF16 && out_dt != LA_F32) return fail(LA_ERR_UNSUPPORTED, "o must be LA_BF16 or LA_F32");
    if (!pow2_in(d_k, 16, 256) || !pow2_in(d_v, 16, 256))
        return fail(LA_ERR_UNSUPPORTED, "d_k and d_v must be 16..256, powers of two");
    la::DeltaStepParams p{};
    p.q = static_cast<const unsigned short*>(q);
    p.k = static_cast<const unsigned short*>(k);
    p.v = static_cast<const unsigned short*>(v);
    p.beta = beta;
    p.alpha = alpha;
    p.S = S;
    p.o = o;
    p.n = n_states;
    p.dk = (int)d_k;
    p.dv = (int)d_v;
    p.out_f32 = out_dt == LA_F32;
    return hip_status(la::run_delta_step(p, (hipStream_t)stream), "delta step launch");
}

}  // extern "C"
