// Kernel parameter blocks and launcher declarations (host and device side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

enum { FMAP_NONE = 0, FMAP_ELU1 = 1 };

// Fused phase 3 (with the carry over the chunks of a group).
struct FwdParams {
    const unsigned short* q;  // [BH, L, dk_g]
    const unsigned short* k;  // [BH, L, dk_g]
    const unsigned short* v;  // [BH, L, dv]
    const unsigned short* k_lo;  // [BH, L, dk_g] bf16 residual of pre-mapped phi(k), or null
    void* o;                  // [BH, L, dv] bf16 or f32
    const float* P0;          // [BH, n_groups * p0_sub, dk_g, dv] exclusive prefixes, or null
    const float* z0;          // [BH, n_groups * p0_sub, dk_g]
    float* S_final;           // [BH, dk_g, dv] or null
    float* z_final;           // [BH, dk_g] or null
    int64_t L;
    int C;          // chunk size, >= 1
    int G;          // chunks per group
    int n_groups;
    int n_dvt;      // column tiles per head
    int dk_g;       // feature width in memory (<= the kernel's DK)
    int dv;         // full value width
    int fmap;       // FMAP_NONE or FMAP_ELU1 (applied to q and k on load)
    float in_scale;
    int normalize;
    int out_f32;
    int xcd_remap;
    int noncausal;  // every row reads P0 (the total state); no intra part, no update
    float out_scale;    // multiplies every output row (identity map with in_scale: s^2)
    float state_scale;  // multiplies the returned final state and normaliser (s)
    int p0_sub;         // prefix slots per group (group g starts at slot g * p0_sub); 0 means 1
    float log2_gamma;   // decayed recurrence S_t = gamma S_{t-1} + k_t^T v_t: log2(gamma) (0: no decay)
};

// Phase 1 (per-chunk states).
struct StatesParams {
    const unsigned short* k;
    const unsigned short* v;
    const unsigned short* k_lo;  // bf16 residual of pre-mapped phi(k), or null
    float* S;      // [BH, n_out, dk_g, dv]
    float* z;      // [BH, n_out, dk_g] or null
    int64_t L;
    int64_t C;     // rows per chunk
    int n_items;   // chunks computed per head
    int n_out;     // chunk stride of S / z per head
    int n_dvt;
    int dk_g;
    int dv;
    int fmap;
    float in_scale;
    int want_z;
    int xcd_remap;
    float log2_gamma;  // decayed recurrence: row r of a chunk ending at e weighs gamma^(e-1-r) (0: no decay)
};

// int8 path: fused phase 3 and phase 1 with exact int32 arithmetic.
struct FwdParamsI8 {
    const signed char* q;
    const signed char* k;
    const signed char* v;
    int* o;            // [BH, L, dv]
    const int* P0;     // [BH, n_groups * p0_sub, dk_g, dv] or null
    int* S_final;      // [BH, dk_g, dv] or null
    int64_t L;
    int C;
    int G;
    int n_groups;
    int n_dvt;
    int dk_g;
    int dv;
    int xcd_remap;
    int noncausal;
    int p0_sub;        // prefix slots per group; 0 means 1
};

struct StatesParamsI8 {
    const signed char* k;
    const signed char* v;
    int* S;        // [BH, n_out, dk_g, dv]
    int* z;        // [BH, n_out, dk_g] or null
    int64_t L;
    int64_t C;
    int n_items;
    int n_out;
    int n_dvt;
    int dk_g;
    int dv;
    int xcd_remap;
};

struct ScanParams {
    void* S;         // [BH, N, E] (E = dk*dv), fp32 or int32
    void* z;         // [BH, N, dk] or null
    void* S_final;   // [BH, E] or null
    void* z_final;   // [BH, dk] or null
    int64_t N;
    int64_t E;
    int64_t Ez;
    int is_int;
    float log2_gamma;  // decayed prefix P_n = gamma^len(n-1) P_{n-1} + S_{n-1} (0: plain sum)
    int64_t L;         // with the decay: rows of the sequence and rows per chunk, so that
    int64_t Cs;        //   len(n) = clamp(L - n Cs, 0, Cs)
};

struct FmapParams {
    const unsigned short* x;  // [rows, d_in]
    const unsigned short* W;  // [m, d_in] or null
    void* y;                  // [rows, d_out] bf16 or f32
    unsigned short* y_lo;     // [rows, d_out] bf16 residual y - bf16(y) (FAVOR+, bf16 y), or null
    int64_t rows;
    int d_in;
    int m;
    int fmap;       // 0 identity (scaled), 1 elu1, 2 favor
    float in_scale;
    int y_f32;
};

struct DecodeParams {
    const unsigned short* q;  // [n, d_in]
    const unsigned short* k;
    const unsigned short* v;  // [n, dv]
    const unsigned short* W;  // [m, d_in] or null
    float* S;                 // [n, dk, dv]
    float* z;                 // [n, dk] or null
    void* o;                  // [n, dv]
    int64_t n;
    int d_in;
    int dk;
    int dv;
    int fmap;       // 0 identity, 1 elu1, 2 favor
    float in_scale;
    int normalize;
    int out_f32;
    float gamma;    // decayed recurrence: S = gamma S + k^T v, z = gamma z + k (1: none)
};

// The delta rule (la_delta.hip).
struct DeltaStepParams {
    const unsigned short* q;  // [n, dk]
    const unsigned short* k;  // [n, dk]
    const unsigned short* v;  // [n, dv]
    const float* beta;        // [n] write strengths
    const float* alpha;       // [n] gates, or null (1)
    float* S;                 // [n, dk, dv], read and updated
    void* o;                  // [n, dv] bf16 or f32
    int64_t n;
    int dk;
    int dv;
    int out_f32;
};

struct DeltaPrepParams {
    const unsigned short* k;  // [BH, L, dk]
    const float* beta;        // [BH, L]
    const float* alpha;       // [BH, L] or null
    unsigned short* T;        // [BH, N, 64, 64] per-chunk transforms (columns in operand order)
    float* lg;                // [BH, N, 64] log2 of the gates' product up to each row of the chunk
    int64_t BH;
    int64_t L;
    int64_t N;                // chunks of 64 rows
    int dk;
};

struct DeltaFwdParams {
    const unsigned short* q;  // [BH, L, dk]
    const unsigned short* k;
    const unsigned short* v;  // [BH, L, dv]
    const unsigned short* T;  // from the transform
    const float* lg;
    unsigned short* o;        // [BH, L, dv] bf16
    float* S_final;           // [BH, dk, dv] or null
    int64_t BH;
    int64_t L;
    int64_t N;
    int dk;
    int dv;
    int n_dvt;                // value tiles of 64 columns
    int xcd_remap;
};

// FAVOR+ mapped inside the streaming kernels (la_favor.hip): 64 input
// features, m in {64, 128, 256} random features, chunks of 64 rows, value
// tiles of 64 columns.
struct FavorParams {
    const unsigned short* q;  // [BH, L, 64] (phase 3)
    const unsigned short* k;  // [BH, L, 64]
    const unsigned short* v;  // [BH, L, dv]
    const unsigned short* W;  // [m, 64]
    unsigned short* o;        // [BH, L, dv] bf16 (phase 3)
    const float* P0;          // phase 3: [BH, n_groups * p0_sub, m, dv] exclusive prefixes, or null
    const float* z0;          // phase 3: [BH, n_groups * p0_sub, m], or null
    float* S;                 // phase 1: [BH, n_out, m, dv]
    float* z;                 // phase 1: [BH, n_out, m] (when the normaliser is wanted)
    int64_t L;
    int64_t rows;             // phase 1: rows per run, a multiple of 64
    int G;                    // phase 3: chunks per group
    int n_groups;             // phase 3: groups per head; phase 1: runs computed per head
    int n_out;                // phase 1: run stride of S and z per head
    int n_dvt;                // value tiles per head
    int dv;
    int p0_sub;               // phase 3: prefix slots per group (group g starts at slot g p0_sub); 0 means 1
    float in_scale;
    int xcd_remap;
};

hipError_t run_favor_states(const FavorParams& p, int m, int norm, int64_t grid, hipStream_t s);
hipError_t run_favor_fwd(const FavorParams& p, int m, int norm, int64_t grid, hipStream_t s);

hipError_t run_delta_step(const DeltaStepParams& p, hipStream_t s);
hipError_t run_delta_transform(const DeltaPrepParams& p, hipStream_t s);
hipError_t run_delta_fwd(const DeltaFwdParams& p, hipStream_t s);

// Log-linear attention: bucket pyramid and the output kernel.
struct LogLinParams {
    const unsigned short* q;  // [BH, L, dk]
    const unsigned short* k;  // [BH, L, dk]
    const unsigned short* v;  // [BH, L, dv]
    const float* lam;         // [BH, L, n_lev] level weights
    const float* S;           // [BH, N, dk, dv] per-chunk states (level-1 buckets)
    const unsigned short* T;  // [BH, n_pyr, dk, dv] bf16 whole-chunk buckets of levels 2.. (or null)
    unsigned short* o;        // [BH, L, dv]
    int64_t L;
    int N;          // chunks
    int n_pyr;      // pyramid nodes per head
    int n_lev;      // levels (1 + bit length of L - 1)
    int n_dvt;
    int dk;
    int dv;
    int xcd_remap;
};

// With lev (the level states after token Tl, n_lev levels), the pyramid nodes
// that are buckets of that state are also written there (fp32).
hipError_t run_loglinear_pyramid(const float* S, unsigned short* T, int64_t BH, int N, int n_pyr, int64_t E,
                                 float* lev, int64_t Tl, int n_lev, hipStream_t s);
hipError_t run_loglinear_fwd(const LogLinParams& p, int64_t grid, hipStream_t s);

// One decode step of log-linear attention over n streams (the Fenwick tree
// recurrence; see loglinear_step_kernel).
struct LogLinStepParams {
    const unsigned short* q;  // [n, dk] bf16
    const unsigned short* k;  // [n, dk] bf16
    const unsigned short* v;  // [n, dv] bf16
    const float* lam;         // [n, n_lev] this token's level weights
    float* S;                 // [n, n_lev, dk, dv] level states, in place
    void* o;                  // [n, dv] f32 or bf16
    int64_t n;
    int64_t t;                // the token's position (>= 0)
    int dk, dv, n_lev;
    int out_f32;
};
hipError_t run_loglinear_step(const LogLinStepParams& p, hipStream_t s);

// The level states a stream holds after its token L - 1 (what L decode steps
// from zero leave), from k, v and the states of its whole 64-row chunks.
struct LogLinPrefixParams {
    const unsigned short* k;  // [BH, L, dk] bf16
    const unsigned short* v;  // [BH, L, dv] bf16
    const float* chunks;      // [BH, n_chunks, dk, dv] per-chunk states (at least the chunks before the last one; or null)
    float* S;                 // [BH, n_lev, dk, dv]
    int64_t BH, L;
    int dk, dv, n_lev, n_chunks;
    int pyr_written;          // levels >= 8 that hold keys were written by the forward's pyramid: left alone
};
hipError_t run_loglinear_prefix_levels(const LogLinPrefixParams& p, hipStream_t s);

hipError_t run_chunked_fwd_i8(const FwdParamsI8& p, int DK, int DVT, int T, int64_t grid, hipStream_t s);
hipError_t run_chunk_states_i8(const StatesParamsI8& p, int DK, int DVT, int64_t grid, hipStream_t s);
// Streaming phase 1 (la_states_pipe.hip): d_k = DK in {64, 128, 256}, value
// tiles of 64 columns, runs of C rows with C a multiple of 64;
// kind 0 plain K, 1 elu+1 applied here (split hi/lo), 2 pre-mapped with residual.
hipError_t states_pipe_bf16(const StatesParams& p, int DK, int kind, int64_t grid, hipStream_t s);
hipError_t run_state_scan(const ScanParams& p, int64_t BH, hipStream_t s);
hipError_t run_feature_map(const FmapParams& p, hipStream_t s);
hipError_t run_recurrent_step(const DecodeParams& p, hipStream_t s);

// One exact int8 decode step: S += k^T v, o = q S in wrapping int32.
struct DecodeParamsI8 {
    const signed char* q;  // [n, dk]
    const signed char* k;  // [n, dk]
    const signed char* v;  // [n, dv]
    int* S;                // [n, dk, dv]
    int* o;                // [n, dv]
    int64_t n;
    int dk, dv;
};
hipError_t run_recurrent_step_i8(const DecodeParamsI8& p, hipStream_t s);

}  // namespace la
