// C ABI of libspecverify: argument validation on the host, then kernel launches on the
// caller's stream.  Every argument error is reported before the first HIP call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/specverify.h"
#include "sv_internal.h"

namespace {

thread_local char g_last_error[256] = "";
// Timing hook: events recorded around the next matmul launch of this thread, then cleared.
thread_local hipEvent_t g_prof_before = nullptr;
thread_local hipEvent_t g_prof_after = nullptr;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other.  Devices are queried once.
std::atomic<int> g_arch[64];

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SV_ERR_DEVICE, "device index %d out of range", dev);
    int known = g_arch[dev].load(std::memory_order_relaxed);
    if (known == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        known = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch[dev].store(known, std::memory_order_relaxed);
    }
    if (known != 1) return fail(SV_ERR_DEVICE, "device %d is not gfx950", dev);
    return SV_OK;
}

int check_q8b32(const int8_t* w, const uint16_t* s, int32_t rows, int32_t H, const uint16_t* x, int32_t S,
                int32_t max_s) {
    if (!w || !s || !x) return fail(SV_ERR_NULL, "weights, scales and activations are required");
    if (rows < 1 || rows > (1 << 30)) return fail(SV_ERR_SHAPE, "rows=%d outside [1, 2^30]", rows);
    if (H < SV_BLOCK || H > 65536 || H % SV_BLOCK) return fail(SV_ERR_SHAPE, "H=%d must be a multiple of 32 in [32, 65536]", H);
    if (S < 1 || S > max_s) return fail(SV_ERR_SHAPE, "S=%d outside [1, %d]", S, max_s);
    if (!aligned(w, 16)) return fail(SV_ERR_ALIGN, "int8 weights must be 16-byte aligned");
    if (!aligned(x, 16)) return fail(SV_ERR_ALIGN, "activation rows must be 16-byte aligned");
    if (!aligned(s, 16)) return fail(SV_ERR_ALIGN, "scales must be 16-byte aligned");
    return SV_OK;
}

// The matmul (and its split combine), timed by the pending hook's events if one is set.
hipError_t launch_matmul(int epi, const sv::GemmCfg& cfg, const sv::GemmArgs& a, hipStream_t stream,
                         bool combine = true) {
    hipEvent_t before = g_prof_before, after = g_prof_after;
    g_prof_before = g_prof_after = nullptr;
    return sv::launch_q8b32(epi, cfg, a, stream, combine, before, after);
}

// The argmax head's matmul under its launch plan: one launch, or two passes over rows 0 .. 31
// and 32 .. S-1 (the hook's events then bracket both).
hipError_t launch_head_matmul(const sv::GemmCfg& cfg, int passes, const sv::GemmArgs& a, hipStream_t stream) {
    if (passes == 1) return launch_matmul(sv::EPI_HEAD, cfg, a, stream);
    hipEvent_t before = g_prof_before, after = g_prof_after;
    g_prof_before = g_prof_after = nullptr;
    sv::GemmArgs lo = a, hi = a;
    lo.S = 32;
    hi.S = a.S - 32;
    hi.x = a.x + (size_t)32 * a.H;
    hi.part_val = a.part_val + (size_t)32 * sv::kGridMax;
    hi.part_idx = a.part_idx + (size_t)32 * sv::kGridMax;
    if (a.logits) hi.logits = a.logits + (size_t)32 * a.V;
    hipError_t e = sv::launch_q8b32(sv::EPI_HEAD, cfg, lo, stream, true, before, nullptr);
    if (e != hipSuccess) return e;
    return sv::launch_q8b32(sv::EPI_HEAD, cfg, hi, stream, true, nullptr, after);
}

// A chunked matmul (head or stack projection), timed by the pending hook's events if one is set.
hipError_t launch_chunked_matmul(int epi, const sv::ChunkCfg& cfg, const sv::ChunkArgs& a, hipStream_t stream) {
    hipEvent_t before = g_prof_before, after = g_prof_after;
    g_prof_before = g_prof_after = nullptr;
    return sv::launch_chunked(epi, cfg, a, stream, before, after);
}

}  // namespace

extern "C" {

const char* specverify_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "null pointer";
        case SV_ERR_SHAPE: return "size out of range";
        case SV_ERR_ALIGN: return "misaligned pointer";
        case SV_ERR_WORKSPACE: return "workspace too small";
        case SV_ERR_CAPACITY: return "token capacity too small";
        case SV_ERR_HIP: return "HIP error";
        case SV_ERR_DEVICE: return "device is not gfx950";
        default: return "unknown status";
    }
}

const char* specverify_last_error(void) { return g_last_error; }

int specverify_profile_next_matmul(hipEvent_t before, hipEvent_t after) {
    if ((before == nullptr) != (after == nullptr)) return fail(SV_ERR_NULL, "give both events or neither");
    g_prof_before = before;
    g_prof_after = after;
    return SV_OK;
}

void specverify_set_tuning(int32_t waves_per_group, int32_t max_groups, int32_t depth, int32_t head_kernel,
                           int32_t split) {
    if (waves_per_group != 0 && waves_per_group != 4 && waves_per_group != 8 && waves_per_group != 16)
        waves_per_group = 0;
    if (max_groups < 0 || max_groups > sv::kGridMax) max_groups = 0;
    if (depth < 0 || depth > 4) depth = 0;
    if (head_kernel < 0 || head_kernel > 3) head_kernel = 0;
    if (split < 0 || split > 8) split = 0;
    sv::set_tuning(waves_per_group, max_groups, head_kernel == 3 ? 1 : 0);
    sv::set_chunk_tuning(waves_per_group, depth, max_groups, head_kernel, split);
}

int specverify_propose(const int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max, int32_t K,
                       int32_t* drafts, hipStream_t stream) {
    if (!tokens || !state || !drafts) return fail(SV_ERR_NULL, "tokens, state and drafts are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (K < 1 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [1, %d]", K, SV_MAX_S - 1);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(tokens, 4) || !aligned(state, 4) || !aligned(drafts, 4)) return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_propose(tokens, cap, state, ngram_max, K, drafts, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "propose launch");
}

size_t specverify_verify_workspace_bytes(int32_t V, int32_t H, int32_t S) {
    if (V < 1 || V > (1 << 30) || H < SV_BLOCK || H > 65536 || H % SV_BLOCK || S < 1 || S > SV_MAX_S) return 0;
    return sv::head_workspace_bytes(V, H, S);
}

namespace {

// Head launch shared by specverify_verify and specverify_round: the matmul writes per-
// workgroup argmax partials (or split sums, then a combine pass reduces them per workgroup),
// and one tail kernel reduces them into argmax[S] and, for a round, accepts and drafts.
int launch_head(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden, int32_t S,
                int32_t* argmax, float* logits, void* workspace, bool round, const int32_t* drafts_in,
                int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts_out,
                hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    float* part_val = reinterpret_cast<float*>(ws);
    int* part_idx = reinterpret_cast<int*>(ws + (size_t)4 * S * sv::kGridMax);
    sv::ChunkCfg cc;
    if (S <= 16 && sv::head_use_chunked(V, H) && sv::chunked_config(V, H, sv::EPI_HEAD, cc)) {
        // ring kernel: argmax partials per workgroup, no hidden-axis split
        sv::ChunkArgs c{};
        c.w0 = wq; c.s0 = wscale; c.x = hidden;
        c.V = V; c.H = H; c.S = S; c.nb = H / SV_BLOCK; c.nitems = cc.items; c.nkc = cc.nkc;
        c.part_val = part_val; c.part_idx = part_idx; c.logits = logits;
        hipError_t e = launch_chunked_matmul(sv::EPI_HEAD, cc, c, stream);
        if (e != hipSuccess) return hip_fail(e, "verify matmul launch");
        e = sv::launch_round_tail(part_val, part_idx, cc.grid, S, argmax, round ? drafts_in : nullptr, tokens, cap,
                                  state, ngram_max, round ? drafts_out : nullptr, stream);
        return e == hipSuccess ? SV_OK : hip_fail(e, "argmax/round tail launch");
    }
    int passes = 1;
    const sv::GemmCfg cfg = sv::head_config(V, H, S, passes);
    sv::GemmArgs a{};
    a.w0 = wq;
    a.s0 = wscale;
    a.x = hidden;
    a.V = V;
    a.H = H;
    a.S = S;
    a.nb = H / SV_BLOCK;
    a.nitems = (V + 15) / 16;
    a.ksplit = cfg.ksplit;
    a.part_val = part_val;
    a.part_idx = part_idx;
    a.logits = logits;
    if (cfg.ksplit > 1) a.kpart0 = reinterpret_cast<float*>(ws + sv::head_partials_bytes(S));
    hipError_t e = launch_head_matmul(cfg, passes, a, stream);
    if (e != hipSuccess) return hip_fail(e, "verify matmul launch");
    const int nparts = cfg.ksplit > 1 ? sv::combine_groups(V) : cfg.grid;
    e = sv::launch_round_tail(a.part_val, a.part_idx, nparts, S, argmax, round ? drafts_in : nullptr, tokens, cap,
                              state, ngram_max, round ? drafts_out : nullptr, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "argmax/round tail launch");
}

int check_head(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden, int32_t S,
               int32_t* argmax, float* logits, void* workspace, size_t workspace_bytes) {
    if (int st = check_q8b32(wq, wscale, V, H, hidden, S, SV_MAX_S)) return st;
    if (!argmax || !workspace) return fail(SV_ERR_NULL, "argmax and workspace are required");
    if (!aligned(argmax, 4) || (logits && !aligned(logits, 4)) || !aligned(workspace, 16))
        return fail(SV_ERR_ALIGN, "argmax/logits 4-byte, workspace 16-byte alignment required");
    const size_t need = sv::head_workspace_bytes(V, H, S);
    if (workspace_bytes < need) return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    return SV_OK;
}

}  // namespace

int specverify_verify(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                      int32_t S, int32_t* argmax, float* logits, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    if (int st = check_head(wq, wscale, V, H, hidden, S, argmax, logits, workspace, workspace_bytes)) return st;
    if (int st = check_device()) return st;
    return launch_head(wq, wscale, V, H, hidden, S, argmax, logits, workspace, false, nullptr, nullptr, 0, nullptr,
                       0, nullptr, stream);
}

int specverify_round(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                     int32_t K, const int32_t* drafts_in, int32_t* tokens, int32_t cap, int32_t* state,
                     int32_t ngram_max, int32_t* drafts_out, int32_t* argmax, float* logits, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    if (K < 1 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [1, %d]", K, SV_MAX_S - 1);
    if (int st = check_head(wq, wscale, V, H, hidden, K + 1, argmax, logits, workspace, workspace_bytes)) return st;
    if (!drafts_in || !tokens || !state || !drafts_out) return fail(SV_ERR_NULL, "drafts, tokens and state are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(drafts_in, 4) || !aligned(tokens, 4) || !aligned(state, 4) || !aligned(drafts_out, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    return launch_head(wq, wscale, V, H, hidden, K + 1, argmax, logits, workspace, true, drafts_in, tokens, cap, state,
                       ngram_max, drafts_out, stream);
}

namespace {

// Scratch of specverify_round_noalloc: the head workspace (per-workgroup argmax partials for
// the largest window; split sums too when a split hidden axis needs them and they fit), in a
// file-scope device array.  Each GPU the library runs on holds its own
// copy until the process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not the device copy): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current, and is kept here.
constexpr size_t kStaticScratchBytes = sv::head_partials_bytes(SV_MAX_S);      // 2 MiB
__device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_addr[64];            // per device; guarded by g_scratch_mu

int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(SV_ERR_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return SV_OK;
}

}  // namespace

int specverify_round_noalloc(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                             const uint16_t* hidden, int32_t K, const int32_t* drafts_in, int32_t* tokens,
                             int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts_out, int32_t* argmax,
                             float* logits, hipStream_t stream) {
    if (K < 1 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [1, %d]", K, SV_MAX_S - 1);
    if (int st = check_q8b32(wq, wscale, V, H, hidden, K + 1, SV_MAX_S)) return st;
    if (!argmax || !drafts_in || !tokens || !state || !drafts_out)
        return fail(SV_ERR_NULL, "argmax, drafts, tokens and state are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(argmax, 4) || (logits && !aligned(logits, 4)) || !aligned(drafts_in, 4) || !aligned(tokens, 4) ||
        !aligned(state, 4) || !aligned(drafts_out, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers and logits must be 4-byte aligned");
    const size_t need = sv::head_workspace_bytes(V, H, K + 1);
    if (need > kStaticScratchBytes)
        return fail(SV_ERR_SHAPE,
                    "V=%d H=%d S=%d needs %zu bytes of scratch (the hidden axis is split across workgroups); the "
                    "library-held scratch holds %zu bytes: use specverify_round with a workspace",
                    V, H, K + 1, need, kStaticScratchBytes);
    if (int st = check_device()) return st;
    void* ws = nullptr;
    if (int st = scratch_address(&ws)) return st;
    return launch_head(wq, wscale, V, H, hidden, K + 1, argmax, logits, ws, true, drafts_in, tokens, cap, state,
                       ngram_max, drafts_out, stream);
}

size_t specverify_sample_workspace_bytes(int32_t V, int32_t H, int32_t S) {
    if (V < 1 || V > (1 << 30) || H < SV_BLOCK || H > 65536 || H % SV_BLOCK || S < 1 || S > 16) return 0;
    return sv::sample_workspace_bytes(V, H, S);
}

namespace {

// Sampling head: the matmul with the sampling epilogue (per-workgroup draw and log-sum-exp
// partials, the draft logits into zd), then the tail that reduces them and, for a round,
// accepts and drafts.  Workspace: [part_val, part_idx][part_m, part_l][zd, 256 B][split sums].
int launch_sample_head(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                       int32_t S, const int32_t* drafts, float temperature, uint64_t seed, int32_t* state,
                       float* zd, int32_t* sample, float* lse, float* logits, void* workspace, bool round,
                       int32_t* tokens, int32_t cap, int32_t ngram_max, int32_t* drafts_out, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    const size_t hp = sv::head_partials_bytes(S);
    const sv::GemmCfg cfg = sv::gemm_config(V, H, S, sv::EPI_SAMPLE);
    sv::GemmArgs a{};
    a.w0 = wq;
    a.s0 = wscale;
    a.x = hidden;
    a.V = V;
    a.H = H;
    a.S = S;
    a.nb = H / SV_BLOCK;
    a.nitems = (V + 15) / 16;
    a.ksplit = cfg.ksplit;
    a.part_val = reinterpret_cast<float*>(ws);
    a.part_idx = reinterpret_cast<int*>(ws + (size_t)4 * S * sv::kGridMax);
    a.part_m = reinterpret_cast<float*>(ws + hp);
    a.part_l = reinterpret_cast<float*>(ws + hp + (size_t)4 * S * sv::kGridMax);
    a.zd = zd ? zd : reinterpret_cast<float*>(ws + 2 * hp);
    a.logits = logits;
    a.state = state;
    a.drafts = drafts;
    a.inv_temp = 1.0f / temperature;
    a.key0 = (uint32_t)seed;
    a.key1 = (uint32_t)(seed >> 32);
    if (cfg.ksplit > 1) a.kpart0 = reinterpret_cast<float*>(ws + 2 * hp + 256);
    hipError_t e = launch_matmul(sv::EPI_SAMPLE, cfg, a, stream);
    if (e != hipSuccess) return hip_fail(e, "sampling verify matmul launch");
    const int nparts = cfg.ksplit > 1 ? sv::combine_groups(V) : cfg.grid;
    e = sv::launch_sample_tail(a.part_val, a.part_idx, a.part_m, a.part_l, nparts, S, V, a.zd, a.key0, a.key1, sample,
                               lse, round ? drafts : nullptr, round ? tokens : nullptr, cap, state, ngram_max,
                               round ? drafts_out : nullptr, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "sampling tail launch");
}

// Checks shared by the generation loops: the token-indexed table and the window it fills.
int check_table(const uint16_t* table, const uint16_t* window, int32_t K, int32_t rounds) {
    if (K < 1 || K > 15) return fail(SV_ERR_SHAPE, "K=%d outside [1, 15]", K);
    if (rounds < 0) return fail(SV_ERR_SHAPE, "rounds=%d < 0", rounds);
    if (!table || !window) return fail(SV_ERR_NULL, "table and window are required");
    if (!aligned(table, 16) || !aligned(window, 16)) return fail(SV_ERR_ALIGN, "table and window must be 16-byte aligned");
    return SV_OK;
}

int check_temperature(float t) {
    if (!(t > 0.0f) || !std::isfinite(t) || !std::isfinite(1.0f / t))
        return fail(SV_ERR_SHAPE, "temperature %g must be positive, finite and have a finite inverse", (double)t);
    return SV_OK;
}

}  // namespace

int specverify_verify_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                             int32_t S, const int32_t* drafts, float temperature, uint64_t seed,
                             const int32_t* state, int32_t* sample, float* lse, float* zd, float* logits,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_q8b32(wq, wscale, V, H, hidden, S, 16)) return st;
    if (int st = check_temperature(temperature)) return st;
    if (!state || !sample || !lse || !zd || !workspace || (S > 1 && !drafts))
        return fail(SV_ERR_NULL, "state, sample, lse, zd, workspace (and drafts when S > 1) are required");
    if (!aligned(state, 4) || !aligned(sample, 4) || !aligned(lse, 4) || !aligned(zd, 4) ||
        (drafts && !aligned(drafts, 4)) || (logits && !aligned(logits, 4)) || !aligned(workspace, 16))
        return fail(SV_ERR_ALIGN, "4-byte aligned buffers and a 16-byte aligned workspace are required");
    const size_t need = sv::sample_workspace_bytes(V, H, S);
    if (workspace_bytes < need) return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    return launch_sample_head(wq, wscale, V, H, hidden, S, drafts, temperature, seed, const_cast<int32_t*>(state),
                              zd, sample, lse, logits, workspace, false, nullptr, 0, 0, nullptr, stream);
}

int specverify_accept_sample(const int32_t* sample, const float* lse, const float* zd, const int32_t* drafts,
                             int32_t K, int32_t V, uint64_t seed, int32_t* tokens, int32_t cap, int32_t* state,
                             hipStream_t stream) {
    if (!sample || !lse || !zd || !tokens || !state || (K > 0 && !drafts))
        return fail(SV_ERR_NULL, "sample, lse, zd, tokens, state (and drafts when K > 0) are required");
    if (K < 0 || K > 15) return fail(SV_ERR_SHAPE, "K=%d outside [0, 15]", K);
    if (V < 1 || V > (1 << 30)) return fail(SV_ERR_SHAPE, "V=%d outside [1, 2^30]", V);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(sample, 4) || !aligned(lse, 4) || !aligned(zd, 4) || !aligned(tokens, 4) || !aligned(state, 4) ||
        (drafts && !aligned(drafts, 4)))
        return fail(SV_ERR_ALIGN, "buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_accept_sample(sample, lse, zd, drafts, K, V, (uint32_t)seed, (uint32_t)(seed >> 32),
                                            tokens, cap, state, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "sampling accept launch");
}

int specverify_round_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                            int32_t K, const int32_t* drafts_in, float temperature, uint64_t seed, int32_t* tokens,
                            int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts_out, int32_t* sample,
                            float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (K < 1 || K > 15) return fail(SV_ERR_SHAPE, "K=%d outside [1, 15]", K);
    if (int st = check_q8b32(wq, wscale, V, H, hidden, K + 1, 16)) return st;
    if (int st = check_temperature(temperature)) return st;
    if (!drafts_in || !tokens || !state || !drafts_out || !workspace)
        return fail(SV_ERR_NULL, "drafts, tokens, state and workspace are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(drafts_in, 4) || !aligned(tokens, 4) || !aligned(state, 4) || !aligned(drafts_out, 4) ||
        (sample && !aligned(sample, 4)) || (lse && !aligned(lse, 4)) || !aligned(workspace, 16))
        return fail(SV_ERR_ALIGN, "4-byte aligned buffers and a 16-byte aligned workspace are required");
    const size_t need = sv::sample_workspace_bytes(V, H, K + 1);
    if (workspace_bytes < need) return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    return launch_sample_head(wq, wscale, V, H, hidden, K + 1, drafts_in, temperature, seed, state, nullptr, sample,
                              lse, nullptr, workspace, true, tokens, cap, ngram_max, drafts_out, stream);
}

int specverify_generate_sample(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                               const uint16_t* table, int32_t K, int32_t rounds, float temperature, uint64_t seed,
                               int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max, int32_t* drafts,
                               uint16_t* window, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_table(table, window, K, rounds)) return st;
    if (int st = check_q8b32(wq, wscale, V, H, window, K + 1, 16)) return st;
    if (int st = check_temperature(temperature)) return st;
    if (!drafts || !tokens || !state || !workspace) return fail(SV_ERR_NULL, "drafts, tokens, state and workspace are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(drafts, 4) || !aligned(tokens, 4) || !aligned(state, 4) || !aligned(workspace, 16))
        return fail(SV_ERR_ALIGN, "4-byte aligned buffers and a 16-byte aligned workspace are required");
    const size_t need = sv::sample_workspace_bytes(V, H, K + 1);
    if (workspace_bytes < need) return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    for (int r = 0; r < rounds; ++r) {
        hipError_t e = sv::launch_gather_window(tokens, cap, state, drafts, K, table, V, H, window, stream);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
        if (int st = launch_sample_head(wq, wscale, V, H, window, K + 1, drafts, temperature, seed, state, nullptr,
                                        nullptr, nullptr, nullptr, workspace, true, tokens, cap, ngram_max, drafts,
                                        stream))
            return st;
    }
    return SV_OK;
}

namespace {

int check_tree_args(int32_t K, int32_t branches, int32_t depth, int32_t ngram_max) {
    if (K < 1 || K > 15) return fail(SV_ERR_SHAPE, "tree nodes K=%d outside [1, 15]", K);
    if (branches < 1 || branches > 4) return fail(SV_ERR_SHAPE, "branches=%d outside [1, 4]", branches);
    if (depth < 1 || depth > K) return fail(SV_ERR_SHAPE, "depth=%d outside [1, K=%d]", depth, K);
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    return SV_OK;
}

}  // namespace

int specverify_propose_tree(const int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max, int32_t K,
                            int32_t branches, int32_t depth, int32_t* parents, int32_t* drafts, hipStream_t stream) {
    if (!tokens || !state || !parents || !drafts) return fail(SV_ERR_NULL, "tokens, state, parents and drafts are required");
    if (int st = check_tree_args(K, branches, depth, ngram_max)) return st;
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(tokens, 4) || !aligned(state, 4) || !aligned(parents, 4) || !aligned(drafts, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_propose_tree(tokens, cap, state, ngram_max, K, branches, depth, parents, drafts, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "tree propose launch");
}

int specverify_accept_tree(const int32_t* argmax, const int32_t* parents, const int32_t* drafts, int32_t K,
                           int32_t* tokens, int32_t cap, int32_t* state, hipStream_t stream) {
    if (!argmax || !parents || !drafts || !tokens || !state)
        return fail(SV_ERR_NULL, "argmax, parents, drafts, tokens and state are required");
    if (K < 1 || K > 15) return fail(SV_ERR_SHAPE, "tree nodes K=%d outside [1, 15]", K);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(argmax, 4) || !aligned(parents, 4) || !aligned(drafts, 4) || !aligned(tokens, 4) ||
        !aligned(state, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_accept_tree(argmax, parents, drafts, K, tokens, cap, state, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "tree accept launch");
}

namespace {

// The tree round's launches (head matmul, then the tree tail); arguments already checked.
int launch_tree_round(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                      int32_t K, const int32_t* parents_in, const int32_t* drafts_in, int32_t* tokens, int32_t cap,
                      int32_t* state, int32_t ngram_max, int32_t branches, int32_t depth, int32_t* parents_out,
                      int32_t* drafts_out, int32_t* argmax, float* logits, void* workspace, hipStream_t stream) {
    const int S = K + 1;
    char* ws = static_cast<char*>(workspace);
    const sv::GemmCfg cfg = sv::gemm_config(V, H, S, sv::EPI_HEAD);
    sv::GemmArgs a{};
    a.w0 = wq;
    a.s0 = wscale;
    a.x = hidden;
    a.V = V;
    a.H = H;
    a.S = S;
    a.nb = H / SV_BLOCK;
    a.nitems = (V + 15) / 16;
    a.ksplit = cfg.ksplit;
    a.part_val = reinterpret_cast<float*>(ws);
    a.part_idx = reinterpret_cast<int*>(ws + (size_t)4 * S * sv::kGridMax);
    a.logits = logits;
    if (cfg.ksplit > 1) a.kpart0 = reinterpret_cast<float*>(ws + sv::head_partials_bytes(S));
    hipError_t e = launch_matmul(sv::EPI_HEAD, cfg, a, stream);
    if (e != hipSuccess) return hip_fail(e, "tree verify matmul launch");
    const int nparts = cfg.ksplit > 1 ? sv::combine_groups(V) : cfg.grid;
    e = sv::launch_tree_tail(a.part_val, a.part_idx, nparts, S, argmax, parents_in, drafts_in, tokens, cap, state,
                             ngram_max, branches, depth, parents_out, drafts_out, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "tree round tail launch");
}

}  // namespace

int specverify_round_tree(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                          int32_t K, const int32_t* parents_in, const int32_t* drafts_in, int32_t* tokens,
                          int32_t cap, int32_t* state, int32_t ngram_max, int32_t branches, int32_t depth,
                          int32_t* parents_out, int32_t* drafts_out, int32_t* argmax, float* logits,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_tree_args(K, branches, depth, ngram_max)) return st;
    if (int st = check_head(wq, wscale, V, H, hidden, K + 1, argmax, logits, workspace, workspace_bytes)) return st;
    if (!parents_in || !drafts_in || !tokens || !state || !parents_out || !drafts_out)
        return fail(SV_ERR_NULL, "tree, tokens and state buffers are required");
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(parents_in, 4) || !aligned(drafts_in, 4) || !aligned(tokens, 4) || !aligned(state, 4) ||
        !aligned(parents_out, 4) || !aligned(drafts_out, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    return launch_tree_round(wq, wscale, V, H, hidden, K, parents_in, drafts_in, tokens, cap, state, ngram_max,
                             branches, depth, parents_out, drafts_out, argmax, logits, workspace, stream);
}

int specverify_generate_tree(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* table,
                             int32_t K, int32_t rounds, int32_t* tokens, int32_t cap, int32_t* state,
                             int32_t ngram_max, int32_t branches, int32_t depth, int32_t* parents, int32_t* drafts,
                             uint16_t* window, int32_t* argmax, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (int st = check_table(table, window, K, rounds)) return st;
    if (int st = check_tree_args(K, branches, depth, ngram_max)) return st;
    if (int st = check_head(wq, wscale, V, H, window, K + 1, argmax, nullptr, workspace, workspace_bytes)) return st;
    if (!parents || !drafts || !tokens || !state) return fail(SV_ERR_NULL, "parents, drafts, tokens and state are required");
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(parents, 4) || !aligned(drafts, 4) || !aligned(tokens, 4) || !aligned(state, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    for (int r = 0; r < rounds; ++r) {
        // a node's row is the row of its own token under the token-indexed model
        hipError_t e = sv::launch_gather_window(tokens, cap, state, drafts, K, table, V, H, window, stream);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
        if (int st = launch_tree_round(wq, wscale, V, H, window, K, parents, drafts, tokens, cap, state, ngram_max,
                                       branches, depth, parents, drafts, argmax, nullptr, workspace, stream))
            return st;
    }
    return SV_OK;
}

namespace {

int check_head_q4(const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                  int32_t S, int32_t* argmax, float* logits, void* workspace, size_t workspace_bytes,
                  sv::Q4Cfg& cfg) {
    if (!wq || !wscale || !hidden || !argmax || !workspace) return fail(SV_ERR_NULL, "weights, scales, hidden, argmax and workspace are required");
    if (V < 1 || V > (1 << 30)) return fail(SV_ERR_SHAPE, "V=%d outside [1, 2^30]", V);
    if (S < 1 || S > 16) return fail(SV_ERR_SHAPE, "S=%d outside [1, 16]", S);
    if (H < 256 || H > 65536 || !sv::q4_config(V, H, cfg))
        return fail(SV_ERR_SHAPE, "H=%d: needs a multiple of 256 that 8 or 16 blocks per wave cover", H);
    if (!aligned(wq, 16) || !aligned(wscale, 16) || !aligned(hidden, 16) || !aligned(workspace, 16) ||
        !aligned(argmax, 4) || (logits && !aligned(logits, 4)))
        return fail(SV_ERR_ALIGN, "codes, scales, hidden and workspace 16-byte; argmax, logits 4-byte");
    if (workspace_bytes < sv::head_partials_bytes(S))
        return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, sv::head_partials_bytes(S));
    return SV_OK;
}

int launch_head_q4(const sv::Q4Cfg& cfg, const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H,
                   const uint16_t* hidden, int32_t S, int32_t* argmax, float* logits, void* workspace, bool round,
                   const int32_t* drafts_in, int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max,
                   int32_t* drafts_out, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    sv::Q4Args a{};
    a.w = wq; a.s = wscale; a.x = hidden;
    a.V = V; a.H = H; a.S = S; a.nb = H / SV_BLOCK; a.nitems = cfg.items;
    a.part_val = reinterpret_cast<float*>(ws);
    a.part_idx = reinterpret_cast<int*>(ws + (size_t)4 * S * sv::kGridMax);
    a.logits = logits;
    hipEvent_t before = g_prof_before, after = g_prof_after;
    g_prof_before = g_prof_after = nullptr;
    hipError_t e = sv::launch_q4(cfg, a, stream, before, after);
    if (e != hipSuccess) return hip_fail(e, "int4 verify matmul launch");
    e = sv::launch_round_tail(a.part_val, a.part_idx, cfg.grid, S, argmax, round ? drafts_in : nullptr, tokens, cap,
                              state, ngram_max, round ? drafts_out : nullptr, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "argmax/round tail launch");
}

}  // namespace

int specverify_verify_q4b32(const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                            int32_t S, int32_t* argmax, float* logits, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    sv::Q4Cfg cfg{};
    if (int st = check_head_q4(wq, wscale, V, H, hidden, S, argmax, logits, workspace, workspace_bytes, cfg)) return st;
    if (int st = check_device()) return st;
    return launch_head_q4(cfg, wq, wscale, V, H, hidden, S, argmax, logits, workspace, false, nullptr, nullptr, 0,
                          nullptr, 0, nullptr, stream);
}

int specverify_round_q4b32(const uint8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* hidden,
                           int32_t K, const int32_t* drafts_in, int32_t* tokens, int32_t cap, int32_t* state,
                           int32_t ngram_max, int32_t* drafts_out, int32_t* argmax, float* logits, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    if (K < 1 || K > 15) return fail(SV_ERR_SHAPE, "K=%d outside [1, 15]", K);
    sv::Q4Cfg cfg{};
    if (int st = check_head_q4(wq, wscale, V, H, hidden, K + 1, argmax, logits, workspace, workspace_bytes, cfg))
        return st;
    if (!drafts_in || !tokens || !state || !drafts_out) return fail(SV_ERR_NULL, "drafts, tokens and state are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(drafts_in, 4) || !aligned(tokens, 4) || !aligned(state, 4) || !aligned(drafts_out, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    return launch_head_q4(cfg, wq, wscale, V, H, hidden, K + 1, argmax, logits, workspace, true, drafts_in, tokens,
                          cap, state, ngram_max, drafts_out, stream);
}

int specverify_gather_window(const int32_t* tokens, int32_t cap, int32_t* state, const int32_t* drafts, int32_t K,
                             const uint16_t* table, int32_t V, int32_t H, uint16_t* window, hipStream_t stream) {
    if (!tokens || !state || !table || !window || (K > 0 && !drafts))
        return fail(SV_ERR_NULL, "tokens, state, drafts, table and window are required");
    if (K < 0 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [0, %d]", K, SV_MAX_S - 1);
    if (V < 1 || V > (1 << 30) || H < SV_BLOCK || H > 65536 || H % SV_BLOCK)
        return fail(SV_ERR_SHAPE, "V=%d H=%d", V, H);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(tokens, 4) || !aligned(state, 4) || (drafts && !aligned(drafts, 4)) || !aligned(table, 16) ||
        !aligned(window, 16))
        return fail(SV_ERR_ALIGN, "int32 buffers 4-byte, table and window 16-byte alignment required");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_gather_window(tokens, cap, state, drafts, K, table, V, H, window, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "gather launch");
}

int specverify_gather_positions(int32_t* state, int32_t cap, const uint16_t* rows, int32_t nrows, int32_t H,
                                int32_t K, uint16_t* window, hipStream_t stream) {
    if (!state || !rows || !window) return fail(SV_ERR_NULL, "state, rows and window are required");
    if (K < 0 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [0, %d]", K, SV_MAX_S - 1);
    if (nrows < 1 || H < SV_BLOCK || H > 65536 || H % SV_BLOCK) return fail(SV_ERR_SHAPE, "nrows=%d H=%d", nrows, H);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(state, 4) || !aligned(rows, 16) || !aligned(window, 16))
        return fail(SV_ERR_ALIGN, "state 4-byte, rows and window 16-byte alignment required");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_gather_positions(state, cap, rows, nrows, H, K + 1, window, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "gather launch");
}

int specverify_generate(const int8_t* wq, const uint16_t* wscale, int32_t V, int32_t H, const uint16_t* table,
                        int32_t K, int32_t rounds, int32_t* tokens, int32_t cap, int32_t* state, int32_t ngram_max,
                        int32_t* drafts, uint16_t* window, int32_t* argmax, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    if (K < 1 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [1, %d]", K, SV_MAX_S - 1);
    if (rounds < 0) return fail(SV_ERR_SHAPE, "rounds=%d < 0", rounds);
    if (!table) return fail(SV_ERR_NULL, "table is required");
    if (!aligned(table, 16)) return fail(SV_ERR_ALIGN, "table must be 16-byte aligned");
    if (int st = check_head(wq, wscale, V, H, window, K + 1, argmax, nullptr, workspace, workspace_bytes)) return st;
    if (!drafts || !tokens || !state) return fail(SV_ERR_NULL, "drafts, tokens and state are required");
    if (ngram_max < 1 || ngram_max > SV_MAX_NGRAM) return fail(SV_ERR_SHAPE, "ngram_max=%d outside [1, %d]", ngram_max, SV_MAX_NGRAM);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(drafts, 4) || !aligned(tokens, 4) || !aligned(state, 4))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    for (int r = 0; r < rounds; ++r) {
        hipError_t e = sv::launch_gather_window(tokens, cap, state, drafts, K, table, V, H, window, stream);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
        if (int st = launch_head(wq, wscale, V, H, window, K + 1, argmax, nullptr, workspace, true, drafts, tokens,
                                 cap, state, ngram_max, drafts, stream))
            return st;
    }
    return SV_OK;
}

int specverify_accept(const int32_t* argmax, const int32_t* drafts, int32_t K, int32_t* tokens, int32_t cap,
                      int32_t* state, hipStream_t stream) {
    if (!argmax || !tokens || !state || (K > 0 && !drafts)) return fail(SV_ERR_NULL, "argmax, drafts, tokens and state are required");
    if (K < 0 || K > SV_MAX_S - 1) return fail(SV_ERR_SHAPE, "K=%d outside [0, %d]", K, SV_MAX_S - 1);
    if (cap < 1) return fail(SV_ERR_CAPACITY, "cap=%d", cap);
    if (!aligned(argmax, 4) || !aligned(tokens, 4) || !aligned(state, 4) || (drafts && !aligned(drafts, 4)))
        return fail(SV_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_accept(argmax, drafts, K, tokens, cap, state, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "accept launch");
}

int specverify_rmsnorm(const uint16_t* x, int32_t S, int32_t H, float eps, uint16_t* y, hipStream_t stream) {
    if (!x || !y) return fail(SV_ERR_NULL, "x and y are required");
    if (S < 1 || S > SV_MAX_S || H < SV_BLOCK || H > 65536 || H % SV_BLOCK) return fail(SV_ERR_SHAPE, "S=%d H=%d", S, H);
    if (!(eps >= 0.0f)) return fail(SV_ERR_SHAPE, "eps must be >= 0");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(SV_ERR_ALIGN, "x and y must be 16-byte aligned");
    if (int st = check_device()) return st;
    hipError_t e = sv::launch_row_norm(nullptr, 0, S, H, x, nullptr, eps, y, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "rmsnorm launch");
}

size_t specverify_stack_workspace_bytes(int32_t N, int32_t Kin, int32_t S, int32_t gateup) {
    if (N < 1 || N > (1 << 30) || Kin < SV_BLOCK || Kin > 65536 || Kin % SV_BLOCK || S < 1 || S > 16) return 0;
    return sv::stack_workspace_bytes(N, Kin, S, gateup != 0);
}

int specverify_gateup_silu_q8b32(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                                 int32_t N, int32_t Kin, const uint16_t* x, int32_t S, uint16_t* m,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_q8b32(wg, sg, N, Kin, x, S, 16)) return st;
    if (!wu || !su || !m) return fail(SV_ERR_NULL, "up weights, scales and output are required");
    if (!aligned(wu, 16) || !aligned(su, 16) || !aligned(m, 2)) return fail(SV_ERR_ALIGN, "alignment");
    const size_t need = sv::stack_workspace_bytes(N, Kin, S, true);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    const sv::GemmCfg cfg = sv::gemm_config(N, Kin, S, sv::EPI_GATEUP);
    sv::GemmArgs a{};
    a.w0 = wg; a.s0 = sg; a.w1 = wu; a.s1 = su; a.x = x;
    a.V = N; a.H = Kin; a.S = S; a.nb = Kin / SV_BLOCK; a.nitems = (N + 7) / 8; a.ksplit = cfg.ksplit;
    a.y = m;
    if (cfg.ksplit > 1) {
        a.kpart0 = static_cast<float*>(workspace);
        a.kpart1 = a.kpart0 + (size_t)cfg.ksplit * S * N;
    }
    hipError_t e = launch_matmul(sv::EPI_GATEUP, cfg, a, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "gate/up launch");
}

int specverify_linear_q8b32(const int8_t* w, const uint16_t* scale, int32_t N, int32_t Kin, const uint16_t* x,
                            int32_t S, const uint16_t* residual, uint16_t* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_q8b32(w, scale, N, Kin, x, S, 16)) return st;
    if (!y) return fail(SV_ERR_NULL, "output is required");
    if (!aligned(y, 2) || (residual && !aligned(residual, 2))) return fail(SV_ERR_ALIGN, "alignment");
    const size_t need = sv::stack_workspace_bytes(N, Kin, S, false);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    const sv::GemmCfg cfg = sv::gemm_config(N, Kin, S, sv::EPI_STORE);
    sv::GemmArgs a{};
    a.w0 = w; a.s0 = scale; a.x = x;
    a.V = N; a.H = Kin; a.S = S; a.nb = Kin / SV_BLOCK; a.nitems = (N + 15) / 16; a.ksplit = cfg.ksplit;
    a.y = y; a.residual = residual;
    if (cfg.ksplit > 1) a.kpart0 = static_cast<float*>(workspace);
    hipError_t e = launch_matmul(sv::EPI_STORE, cfg, a, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "linear launch");
}

int specverify_linear_residual_rmsnorm_q8b32(const int8_t* w, const uint16_t* scale, int32_t N, int32_t Kin,
                                             const uint16_t* x, int32_t S, const uint16_t* residual, uint16_t* y,
                                             float eps, uint16_t* norm_out, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    if (int st = check_q8b32(w, scale, N, Kin, x, S, 16)) return st;
    if (!y || !norm_out) return fail(SV_ERR_NULL, "y and norm_out are required");
    if (!(eps >= 0.0f)) return fail(SV_ERR_SHAPE, "eps must be >= 0");
    if (!aligned(y, 2) || !aligned(norm_out, 2) || (residual && !aligned(residual, 2)))
        return fail(SV_ERR_ALIGN, "alignment");
    if (norm_out == y || norm_out == residual || norm_out == x)
        return fail(SV_ERR_SHAPE, "norm_out must not alias x, y or residual");
    const size_t need = sv::stack_workspace_bytes(N, Kin, S, false);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;
    const sv::GemmCfg cfg = sv::gemm_config(N, Kin, S, sv::EPI_STORE);
    sv::GemmArgs a{};
    a.w0 = w; a.s0 = scale; a.x = x;
    a.V = N; a.H = Kin; a.S = S; a.nb = Kin / SV_BLOCK; a.nitems = (N + 15) / 16; a.ksplit = cfg.ksplit;
    a.y = y; a.residual = residual;
    if (cfg.ksplit > 1) a.kpart0 = static_cast<float*>(workspace);
    // split: the row pass sums the partials, adds the residual and normalises in one launch;
    // unsplit: the matmul epilogue adds the residual and the row pass only normalises y
    const bool fused = cfg.ksplit > 1 && cfg.ksplit <= sv::kRowNormMaxSplit;
    hipError_t e = launch_matmul(sv::EPI_STORE, cfg, a, stream, /*combine=*/!fused);
    if (e != hipSuccess) return hip_fail(e, "linear launch");
    e = fused ? sv::launch_row_norm(a.kpart0, cfg.ksplit, S, N, residual, y, eps, norm_out, stream)
                       : sv::launch_row_norm(nullptr, 0, S, N, y, nullptr, eps, norm_out, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "row norm launch");
}

namespace {

// Workspace of specverify_stack: m = silu(g) * u [S][F] fp16, then the sum-of-squares
// partials [S][H/16] fp32, then (when the down projection splits its hidden axis ks ways) its
// fp32 slice sums [ks][S][H] and one arrival counter per 16-row tile; each part 256-byte
// aligned.
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t stack_m_bytes(int S, int F) { return align256((size_t)2 * S * F); }
size_t stack_ss_bytes(int S, int H) { return align256((size_t)4 * S * (H / 16)); }

bool stack_shape_ok(int H, int F) {
    sv::ChunkCfg c;
    return H >= 512 && F >= 512 && H <= 65536 && F <= 65536 && H % 512 == 0 && F % 512 == 0 &&
           sv::chunked_config(F, H, sv::EPI_GATEUP, c) && sv::chunked_config(H, F, sv::EPI_STORE, c);
}

}  // namespace

size_t specverify_stack_forward_workspace_bytes(int32_t H, int32_t F, int32_t S) {
    if (S < 1 || S > 16 || !stack_shape_ok(H, F)) return 0;
    return stack_m_bytes(S, F) + stack_ss_bytes(S, H) + sv::chunked_split_bytes(H, F, S);
}

int specverify_stack(const int8_t* wg, const uint16_t* sg, const int8_t* wu, const uint16_t* su,
                     const int8_t* wd, const uint16_t* sd, int32_t L, int32_t H, int32_t F, uint16_t* x,
                     int32_t S, float eps, uint16_t* x_layers, uint16_t* norm_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    if (!wg || !sg || !wu || !su || !wd || !sd || !x || !norm_out || !workspace)
        return fail(SV_ERR_NULL, "weights, scales, x, norm_out and workspace are required");
    if (L < 1 || L > 4096) return fail(SV_ERR_SHAPE, "L=%d outside [1, 4096]", L);
    if (S < 1 || S > 16) return fail(SV_ERR_SHAPE, "S=%d outside [1, 16]", S);
    if (!stack_shape_ok(H, F))
        return fail(SV_ERR_SHAPE, "H=%d and F=%d must be multiples of 512 in [512, 65536] with H*F < 2^31", H, F);
    if (!(eps >= 0.0f)) return fail(SV_ERR_SHAPE, "eps must be >= 0");
    const void* ptrs16[] = {wg, sg, wu, su, wd, sd, x, norm_out, workspace};
    for (const void* p : ptrs16)
        if (!aligned(p, 16)) return fail(SV_ERR_ALIGN, "all buffers must be 16-byte aligned");
    if (x_layers && !aligned(x_layers, 16)) return fail(SV_ERR_ALIGN, "x_layers must be 16-byte aligned");
    const size_t rows_bytes = (size_t)2 * S * H;
    auto overlaps = [](const void* p, size_t pn, const void* q, size_t qn) {
        const char* a = static_cast<const char*>(p);
        const char* b = static_cast<const char*>(q);
        return a < b + qn && b < a + pn;
    };
    if (overlaps(norm_out, rows_bytes, x, rows_bytes) ||
        (x_layers && (overlaps(norm_out, rows_bytes, x_layers, rows_bytes * L) ||
                      overlaps(x, rows_bytes, x_layers, rows_bytes * L))))
        return fail(SV_ERR_SHAPE, "norm_out, x and x_layers must not overlap");
    const size_t need = specverify_stack_forward_workspace_bytes(H, F, S);
    if (workspace_bytes < need) return fail(SV_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (int st = check_device()) return st;

    sv::ChunkCfg cg, cd;
    sv::chunked_config(F, H, sv::EPI_GATEUP, cg);
    sv::chunked_config(H, F, sv::EPI_STORE, cd, S);
    uint16_t* m = static_cast<uint16_t*>(workspace);
    float* ss = reinterpret_cast<float*>(static_cast<char*>(workspace) + stack_m_bytes(S, F));
    float* kpart = nullptr;
    uint32_t* counters = nullptr;
    if (cd.ks > 1) {
        char* split = static_cast<char*>(workspace) + stack_m_bytes(S, F) + stack_ss_bytes(S, H);
        kpart = reinterpret_cast<float*>(split);
        counters = reinterpret_cast<uint32_t*>(split + align256((size_t)4 * cd.ks * S * H));
    }

    // the first pass also clears the tile counters (each down launch leaves them at zero)
    hipError_t e = sv::launch_row_ss(x, S, H, ss, counters, counters ? cd.items : 0, stream);
    if (e != hipSuccess) return hip_fail(e, "row sum-of-squares launch");
    const uint16_t* cur = x;
    for (int l = 0; l < L; ++l) {
        uint16_t* out = x_layers ? x_layers + (size_t)l * S * H : x;
        sv::ChunkArgs g{};
        g.w0 = wg + (size_t)l * F * H;
        g.s0 = sg + (size_t)l * F * (H / SV_BLOCK);
        g.w1 = wu + (size_t)l * F * H;
        g.s1 = su + (size_t)l * F * (H / SV_BLOCK);
        g.x = cur;
        g.norm_ss = ss;
        g.norm_tiles = H / 16;
        g.eps = eps;
        g.V = F; g.H = H; g.S = S; g.nb = H / SV_BLOCK; g.nitems = cg.items; g.nkc = cg.nkc;
        g.y = m;
        e = launch_chunked_matmul(sv::EPI_GATEUP, cg, g, stream);
        if (e != hipSuccess) return hip_fail(e, "stack gate/up launch");
        sv::ChunkArgs d{};
        d.w0 = wd + (size_t)l * H * F;
        d.s0 = sd + (size_t)l * H * (F / SV_BLOCK);
        d.x = m;
        d.V = H; d.H = F; d.S = S; d.nb = F / SV_BLOCK; d.nitems = cd.items; d.nkc = cd.nkc;
        d.y = out;
        d.residual = cur;
        d.ss_out = ss;
        d.kslices = cd.ks;
        d.kpart = kpart;
        d.counters = counters;
        e = launch_chunked_matmul(sv::EPI_STORE, cd, d, stream);
        if (e != hipSuccess) return hip_fail(e, "stack down launch");
        cur = out;
    }
    e = sv::launch_apply_norm(cur, ss, S, H, eps, norm_out, stream);
    return e == hipSuccess ? SV_OK : hip_fail(e, "final norm launch");
}

}  // extern "C"
