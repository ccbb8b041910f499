// Host-side internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Launch `fn`; when a start or stop event is given, the events take the timestamps of this
// kernel's own dispatch packet (the same clock a kernel trace reads), not of a marker
// enqueued before or after it.
template <typename F, typename... Args>
inline void launch_timed(F fn, dim3 grid, dim3 block, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                         Args... args) {
    if (start || stop)
        hipExtLaunchKernelGGL(fn, grid, block, 0, stream, start, stop, 0, args...);
    else
        hipLaunchKernelGGL(fn, grid, block, 0, stream, args...);
}


// EPI_SAMPLE: the head epilogue of sampling verify (per-row log-normaliser, a Gumbel-max
// draw per row that leaves out the row's draft, the scaled logit of that draft).
enum Epi { EPI_HEAD = 0, EPI_STORE = 1, EPI_GATEUP = 2, EPI_SAMPLE = 3 };

constexpr int kGridMax = 4096;     // upper bound on workgroups of one q8b32 launch

// Launch shape of one q8b32 matmul, a pure function of (rows, H, S, tuning).
struct GemmCfg {
    int mt;       // 16-row M tiles of the window: 1, 2 or 4
    int nbw;      // hidden blocks held per wave (register budget bucket)
    int nw;       // waves per workgroup (in-workgroup split of the hidden axis)
    int ksplit;   // split of the hidden axis across workgroups (>1 only for very long H)
    int grid;     // workgroups along the row axis
    int fast;     // 1: 128-byte-segment loads with an LDS exchange; 0: generic loads
    int xr;       // head, mt = 1: window rows beyond the 16-row tile handled by dot products
                  // from LDS (1 for a 17-row window), 0 otherwise
    int xcd;      // 1: items in one contiguous range per die (item_range in sv_gemm.hip), grid a
                  // multiple of 8
};

// epi = the epilogue kind (Epi); the stack epilogues take S <= 16.
GemmCfg gemm_config(int rows, int H, int S, int epi);
// Launch plan of the argmax head: passes = 2 runs a window of more than 32 rows as two passes
// of the returned two-tile configuration (rows 0 .. 31, then 32 .. S-1), each writing complete
// argmax partials for its own rows; passes = 1 is one launch of the returned configuration.
GemmCfg head_config(int V, int H, int S, int& passes);
// Workgroups of the split-combine pass (also the number of argmax partials it writes).
int combine_groups(int V);
void set_tuning(int waves_per_group, int max_groups, int no_extra_row);
// The calling thread's overrides (0 = automatic): waves per workgroup, workgroups per launch.
int tuning_waves();
int tuning_groups();

struct GemmArgs {
    const int8_t* w0;
    const uint16_t* s0;
    const int8_t* w1;          // EPI_GATEUP: up projection
    const uint16_t* s1;
    const uint16_t* x;         // [S][H] fp16
    int V, H, S, nb, nitems, ksplit;
    float* part_val;           // EPI_HEAD: per-workgroup argmax partials [S][kGridMax]
    int* part_idx;
    float* logits;             // EPI_HEAD: [S][V] or null
    uint16_t* y;               // EPI_STORE / EPI_GATEUP: [S][V] fp16
    const uint16_t* residual;  // EPI_STORE: [S][V] fp16 or null
    float* kpart0;             // ksplit > 1: fp32 partial sums [ksplit][S][V]
    float* kpart1;             // ksplit > 1, EPI_GATEUP: partial sums of the up projection
    // EPI_SAMPLE (S <= 16): z = L * inv_temp; row s leaves out draft drafts[s] (s < S-1) from
    // its draw; part_val/part_idx then hold the best Gumbel key and its id, part_m/part_l the
    // running max of z and the sum of exp(z - max); zd[s] = z of draft drafts[s].
    const int32_t* state;      // round state: state[0] = P0, the position row 0 predicts
    const int32_t* drafts;     // [S-1] or null (S = 1)
    float inv_temp;
    uint32_t key0, key1;       // Philox key = the 64-bit seed
    int xcd;                   // item order of the argmax head (GemmCfg::xcd), set by the launcher;
                               // it fills the padding before the next pointer
    float* part_m;             // [S][kGridMax]
    float* part_l;
    float* zd;                 // [S]
};

// Head workspace layout: per-workgroup argmax partials [S][kGridMax] (values, then indices),
// then the split sums when the hidden axis is split across workgroups.
constexpr size_t head_partials_bytes(int S) { return (size_t)8 * S * kGridMax; }
// Sampling head: the head layout, then part_m, part_l [S][kGridMax] and zd [S] (256-byte
// aligned blocks).
size_t sample_workspace_bytes(int V, int H, int S);
// Draw stage 2 of a sampling head launch (per-row draw, log-normaliser) and, when tokens !=
// null, the sampling accept and the next drafts: one workgroup.  sample_out / lse_out may be
// null in a round.
hipError_t launch_sample_tail(const float* pv, const int* pi, const float* pm, const float* pl, int nparts, int S,
                              int V, const float* zd, uint32_t key0, uint32_t key1, int32_t* sample_out,
                              float* lse_out, const int32_t* drafts_in, int32_t* tokens, int cap, int32_t* state,
                              int nmax, int32_t* drafts_out, hipStream_t stream);
hipError_t launch_accept_sample(const int32_t* sample, const float* lse, const float* zd, const int32_t* drafts,
                                int K, int V, uint32_t key0, uint32_t key1, int32_t* tokens, int cap,
                                int32_t* state, hipStream_t stream);

// Tree verify (sv_tree.hip), K <= 15 draft nodes: the round tail after a head matmul
// (argmax, the walk down the tree, the next tree), and the standalone drafter and walk.
hipError_t launch_tree_tail(const float* pv, const int* pi, int nparts, int S, int32_t* argmax,
                            const int32_t* parents_in, const int32_t* drafts_in, int32_t* tokens, int cap,
                            int32_t* state, int nmax, int branches, int depth, int32_t* parents_out,
                            int32_t* drafts_out, hipStream_t stream);
hipError_t launch_propose_tree(const int32_t* tokens, int cap, int32_t* state, int nmax, int K, int branches,
                               int depth, int32_t* parents_out, int32_t* drafts_out, hipStream_t stream);
hipError_t launch_accept_tree(const int32_t* argmax, const int32_t* parents, const int32_t* drafts, int K,
                              int32_t* tokens, int cap, int32_t* state, hipStream_t stream);

// Workspace bytes a head matmul of this shape needs.
size_t head_workspace_bytes(int V, int H, int S);
// Workspace bytes a store / gate-up matmul needs (non-zero only when ksplit > 1).
size_t stack_workspace_bytes(int N, int K, int S, bool gateup);

// The matmul and, when cfg.ksplit > 1 and `combine` is set, the pass that sums the split
// partial sums into the epilogue's output.  `start` / `stop` (optional) time the matmul's
// dispatch through the combine pass.
hipError_t launch_q8b32(int epi, const GemmCfg& cfg, const GemmArgs& a, hipStream_t stream, bool combine = true,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Argmax stage 2 of a head launch and, when drafts_out != null, the rest of the round
// (accept, then the next drafts): one workgroup.
hipError_t launch_round_tail(const float* pv, const int* pi, int nparts, int S, int32_t* argmax,
                             const int32_t* drafts_in, int32_t* tokens, int cap, int32_t* state, int nmax,
                             int32_t* drafts_out, hipStream_t stream);
hipError_t launch_propose(const int32_t* tokens, int cap, int32_t* state, int nmax, int K, int32_t* drafts,
                          hipStream_t stream);
// Window rows [tokens[len-1], drafts (pads -> 0)] of a token-indexed table [V][H] into out [K+1][H].
hipError_t launch_gather_window(const int32_t* tokens, int cap, int32_t* state, const int32_t* drafts, int K,
                                const uint16_t* table, int V, int H, uint16_t* out, hipStream_t stream);
// Window rows [rows[len-1], ..., rows[len-1+S-1]] of a position-indexed model [nrows][H] into out [S][H].
hipError_t launch_gather_positions(int32_t* state, int cap, const uint16_t* rows, int nrows, int H, int S,
                                   uint16_t* out, hipStream_t stream);
hipError_t launch_accept(const int32_t* argmax, const int32_t* drafts, int K, int32_t* tokens,
                         int cap, int32_t* state, hipStream_t stream);
// Per window row: t = sum of `ks` split partial sums [ks][S][N] (+ residual), y = fp16(t)
// (y may be null), norm_out = fp16(RMSNorm(fp16(t))).  ks = 0 is a plain RMSNorm of residual.
constexpr int kRowNormMaxSplit = 8;
hipError_t launch_row_norm(const float* part, int ks, int S, int N, const uint16_t* residual, uint16_t* y,
                           float eps, uint16_t* norm_out, hipStream_t stream);

// Int4 per-block-32 head matmul with the argmax epilogue (sv_q4.hip).  Window rows S <= 16.
struct Q4Args {
    const uint8_t* w;          // [V][H/2] packed codes
    const uint16_t* s;         // [V][H/32] fp16 scales
    const uint16_t* x;         // [S][H] fp16 window rows
    int V, H, S, nb, nitems;
    float* part_val;           // per-workgroup argmax partials [S][kGridMax]
    int* part_idx;
    float* logits;             // [S][V] or null
};
struct Q4Cfg {
    int nbw, nw, grid, items;
};
bool q4_config(int V, int H, Q4Cfg& c);
hipError_t launch_q4(const Q4Cfg& c, const Q4Args& a, hipStream_t stream, hipEvent_t start = nullptr,
                     hipEvent_t stop = nullptr);

// Chunked streaming matmul (dense stack, and heads whose hidden axis splits into whole 128-byte
// wave segments): see sv_chunked.hip.  Window rows S <= 16.
struct ChunkArgs {
    const int8_t* w0;          // [V][H] (gate rows for EPI_GATEUP)
    const uint16_t* s0;
    const int8_t* w1;          // EPI_GATEUP: up projection
    const uint16_t* s1;
    const uint16_t* x;         // [S][H] fp16 window rows (before the norm when norm_ss is set)
    const float* norm_ss;      // [S][norm_tiles] sum-of-squares partials of x, or null (no norm)
    int norm_tiles;
    float eps;
    int V, H, S, nb, nitems, nkc;
    float* part_val;           // EPI_HEAD: per-workgroup argmax partials [S][kGridMax]
    int* part_idx;
    float* logits;             // EPI_HEAD: [S][V] or null
    uint16_t* y;               // EPI_STORE / EPI_GATEUP: [S][V] fp16
    const uint16_t* residual;  // EPI_STORE: [S][V] fp16 or null
    float* ss_out;             // EPI_STORE: [S][nitems] sum of squares of each stored 16-column tile, or null
    // EPI_STORE with the hidden axis split across workgroups (kslices > 1): workgroup b works on
    // slice b / (grid / kslices) of the hidden axis, writes its fp32 tile sums to kpart
    // [kslices][S][V], and the last of a tile's kslices workgroups to finish (counted in
    // counters[tile], which must be zero at launch and is left zero) adds them in slice order
    // and runs the epilogue.
    int kslices;
    float* kpart;
    uint32_t* counters;
};
struct ChunkCfg {
    int nw;       // waves per workgroup (4 .. 16)
    int nkc;      // hidden-axis chunks per tile (chunk = nw x 128 bytes)
    int hold;     // nkc when the window rows stay in registers (nkc <= 2), else 0 (streamed with each unit)
    int depth;    // load units in flight per wave
    int grid;     // workgroups
    int items;    // tiles (16 rows; gate/up: 8 row pairs)
    int ks;       // EPI_STORE: slices of the hidden axis across workgroups (1: none); nkc and hold
                  // then describe one slice
};
// split = 0 or 1: a store projection's hidden axis is not split (the automatic choice); k > 1:
// split k ways when a held-row shape exists for that k (else unsplit).
void set_chunk_tuning(int waves, int depth, int max_groups, int head_kernel, int split);
// Bytes of the split partial sums and tile counters a store projection of this shape needs
// (0 when its configuration does not split).
size_t chunked_split_bytes(int rows, int H, int S);
// Whether the head matmul of this shape runs on the chunked ring kernel (when it applies).
bool head_use_chunked(int V, int H);
// False when H is not a whole number of 4-block segments for 4, 8 or 16 waves.  S > 0 lets a
// store projection split its hidden axis across workgroups when the calling thread's tuning
// asks for it (the split's workspace depends on S).
bool chunked_config(int rows, int H, int epi, ChunkCfg& c, int S = 0);
hipError_t launch_chunked(int epi, const ChunkCfg& c, const ChunkArgs& a, hipStream_t stream,
                          hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// ss[s][t] = sum of squares of the 16 fp16 values of x[s][16t .. 16t+15]; also zeroes
// zero[0 .. nzero) when zero is given.
hipError_t launch_row_ss(const uint16_t* x, int S, int H, float* ss, uint32_t* zero, int nzero,
                         hipStream_t stream);
// out = fp16(x * inv[s]), inv from the ss partials as the chunked gate/up prologue computes it
hipError_t launch_apply_norm(const uint16_t* x, const float* ss, int S, int H, float eps, uint16_t* out,
                             hipStream_t stream);

}  // namespace sv
