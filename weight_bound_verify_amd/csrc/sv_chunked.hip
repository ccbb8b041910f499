// Chunked streaming q8b32 matmul for the weight-bound dense stack, and the row passes that
// carry its RMSNorm between layers.
//
// Page: "Flagship dramatic-speedup plan - the full stackable tuning set", sections "Baseline
// byte model" (a decode step reads every weight byte once; its time is bytes / bandwidth) and
// "Axis 4" (the RMSNorm fused into the neighbouring kernels).  The contraction and its MFMA
// mapping are those of the head matmul (int8 codes of one 32-block -> exact fp16, one
// v_mfma_f32_16x16x32_f16 per block and 16 rows, block scale applied in fp32):
//   out[s, v] = sum_b f32(scale[v, b]) * sum_{k in block b} f32(w[v, k]) * f32(x[s, k])
//
// Why another kernel: a stack projection streams only 50-110 MB, so a launch lasts 10-25 us
// and its ramp-up and drain are a large share of it.  Here a workgroup of NW waves walks a
// flat sequence of load units, one unit = one 16-row tile x one chunk of the hidden axis in
// which every wave owns one 128-byte segment (4 blocks) of each of the 16 rows.  Each wave
// keeps DEPTH units in flight in a ring of registers and issues the next unit as soon as it
// has consumed one, so loads leave at an even rate from the first to the last unit; the
// per-tile cross-wave reduction happens after the tile's last chunk.  The window rows are
// held in registers for the whole launch when the hidden axis has at most two chunks
// (HOLD), and are otherwise loaded with each unit from L2 (they are a few hundred KB, read
// by every workgroup).
//
// The stack's RMSNorm never gets a launch of its own: the down projection's epilogue adds
// the residual, stores the fp16 stream and writes, per 16-column tile, the sum of squares
// of the stored values; the next gate/up launch reduces those partials in a fixed order to
// 1/sqrt(mean + eps) per row and normalises its window rows as it loads them.
#include "sv_device.h"
#include "sv_internal.h"

#include <climits>
#include <cmath>
#include <mutex>

namespace sv {

namespace {

constexpr int kUnitBytes = 2048;        // one wave's unit: 16 rows x 128 bytes
constexpr int kMaxSlices = 8;           // most slices a store projection's hidden axis splits into
constexpr int kMaxSliceItems = 64;      // most tiles one workgroup of a split launch takes

__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Tile row n (0..15) of item `it`: 16 rows of one matrix, or for gate/up 8 gate rows (n < 8)
// and the same 8 rows of the up matrix (n >= 8).
template <int EPI>
__device__ __forceinline__ int crow(int it, int n) {
    return EPI == EPI_GATEUP ? it * 8 + (n & 7) : it * kTileRows + n;
}

// 1 / sqrt(sum_t ss[s][t] / H + eps) for the window rows s of this workgroup, summed in one
// fixed order: lane l folds partials 4l .. 4l+3, then 256 + 4l .. 256 + 4l + 3, ... in
// sequence, then the lanes fold with a fixed butterfly.  Every workgroup and the final norm
// pass use this order, so they get the same value.  Written to inv[s].
template <int NW>
__device__ __forceinline__ void norm_scales(const float* __restrict__ ss, int nt, int S, int H, float eps, int wave,
                                            int lane, float* inv) {
    for (int s = wave; s < S; s += NW) {
        float t = 0.f;
        for (int base = 0; base < nt; base += 4 * kWave) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = base + 4 * lane + e;
                v[e] = i < nt ? ss[(size_t)s * nt + i] : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) t += v[e];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, kWave);
        if (lane == 0) inv[s] = 1.0f / sqrtf(t / (float)H + eps);
    }
}

__device__ __forceinline__ f16x8 scale_f16x8(f16x8 h, float f) {
    f16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)((float)h[e] * f);
    return r;
}

// Raw buffer view of `bytes` bytes at p: 32-bit offsets from a scalar base, and loads past
// the end return zeros (tail rows of the last tile need no clamping).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_view(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr int kAuxNT = 2;        // non-temporal: the weights are read once
// Device-coherent access (the sc1 cache-policy bit): a store is acknowledged only once it is
// visible to every compute unit of the device, and a load reads the device-coherent copy.
// The split fold exchanges its fp32 shares this way instead of writing back and invalidating
// whole caches.
constexpr int kAuxDevice = 16;
constexpr uint32_t kPastEnd = 0xF0000000u;   // an offset beyond every view (views are < 2^31 bytes)

template <int HOLD>
struct Unit {
    u32x4 w[2];                       // [row half]: 16 bytes of rows 8h + lane/8
    u32x2 sc, sc2;                    // fp16 scales of the lane's row, 4 blocks (gate/up: gate | up, one is zero)
    f16x8 hid[HOLD ? 1 : 4];          // window rows of the unit's 4 blocks (streamed mode)
};
// Nothing is computed from a unit's registers until the unit is consumed: an instruction
// that used a just-issued load would wait for every older load too.

// Every wave issues the same sequence of memory instructions whatever the data: loads past a
// workgroup's last unit and stores of rows past S read zeros / are dropped by the buffer
// bounds check instead of being skipped by a branch.  The compiler's wait counts are then
// exact, so waiting for the oldest unit of the ring never drains the younger ones.
//
// HOLD = 1 or 2: the hidden axis has exactly HOLD chunks, the window rows stay in registers,
// and one ring cycle of DEPTH units covers DEPTH / HOLD whole tiles.  HOLD = 0: any number of
// chunks (a multiple of DEPTH), window rows loaded with each unit, one cycle = DEPTH chunks of
// one tile.
template <int NW, int DEPTH, int HOLD, int EPI>
__global__ __launch_bounds__(NW * 64) void q8b32_chunked(ChunkArgs a) {
    static_assert(HOLD == 0 || DEPTH % HOLD == 0, "a ring cycle must cover whole tiles");
    static_assert(NW >= 1 && NW <= 16, "1 .. 16 waves");
    constexpr int RPW = (16 + NW - 1) / NW;       // window rows each wave finishes per tile (rows >= 16 idle)
    __shared__ f32x4 red[2][NW][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xch[NW][2][kUnitBytes];
    __shared__ float inv_s[kTileRows];
    __shared__ int fold_it[kMaxSliceItems];
    __shared__ int fold_n;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int lrow = lane >> 3, lchunk = lane & 7;
    const int nkc = HOLD ? HOLD : a.nkc;
    // Split store projection: the grid is kslices x gps workgroups; workgroup b takes slice
    // b / gps of the hidden axis (nkc chunks from block kbase on) and the tiles r, r + gps, ...
    // with r = b % gps.  Unsplit: one slice, r = b, and the tiles b, b + grid, ...
    const int ks = EPI == EPI_STORE && a.kslices > 1 ? a.kslices : 1;
    const int step = (int)gridDim.x / ks;
    const int slice = ks > 1 ? (int)blockIdx.x / step : 0;
    const int first = (int)blockIdx.x - slice * step;
    const int kbase = slice * nkc * NW * 4;
    const int my_items = first < a.nitems ? (a.nitems - 1 - first) / step + 1 : 0;
    const bool row_ok = n < a.S;       // lanes whose A-operand row is a real window row

    const uint32_t wbytes = (uint32_t)a.V * (uint32_t)a.H;
    const uint32_t sbytes = (uint32_t)a.V * (uint32_t)a.nb * 2u;
    const __amdgpu_buffer_rsrc_t rw0 = buf_view(a.w0, wbytes), rs0 = buf_view(a.s0, sbytes);
    const __amdgpu_buffer_rsrc_t rw1 = buf_view(EPI == EPI_GATEUP ? a.w1 : a.w0, wbytes);
    const __amdgpu_buffer_rsrc_t rs1 = buf_view(EPI == EPI_GATEUP ? a.s1 : a.s0, sbytes);
    const __amdgpu_buffer_rsrc_t rx = buf_view(a.x, (uint32_t)a.S * (uint32_t)a.H * 2u);
    // per-lane parts of the offsets: weight row within the tile half, window row
    const uint32_t wlane = (uint32_t)lrow * (uint32_t)a.H + 16u * lchunk;
    const uint32_t xlane = row_ok ? ((uint32_t)n * (uint32_t)a.H + 8u * g) * 2u : kPastEnd;  // rows >= S read zeros
    const bool srow_up = EPI == EPI_GATEUP && n >= 8;

    // Unit (k-th tile of this workgroup, chunk c); k >= my_items loads zeros.
    auto load = [&](Unit<HOLD>& r, int k, int c) {
        const bool live = k < my_items;
        const int it = first + k * step;
        const int blk0 = kbase + c * (NW * 4) + wave * 4;
        // tile half h covers weight rows base_h .. base_h + 7 (gate/up: 8 gate rows, then the same 8 up rows)
        const uint32_t base0 = (uint32_t)(EPI == EPI_GATEUP ? it * 8 : it * kTileRows);
        const uint32_t base1 = EPI == EPI_GATEUP ? base0 : base0 + 8u;
        const uint32_t kofs = (uint32_t)blk0 * kBlock;
        const uint32_t o0 = live ? base0 * (uint32_t)a.H + kofs + wlane : kPastEnd;
        const uint32_t o1 = live ? base1 * (uint32_t)a.H + kofs + wlane : kPastEnd;
        r.w[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw0, (int)o0, 0, kAuxNT));
        r.w[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw1, (int)o1, 0, kAuxNT));
        const uint32_t srow = (uint32_t)crow<EPI>(it, n);
        const uint32_t sofs = live ? (srow * (uint32_t)a.nb + (uint32_t)blk0) * 2u : kPastEnd;
        if constexpr (EPI == EPI_GATEUP) {
            // both descriptors stay uniform: each lane reads its own matrix and gets zeros
            // (an offset past the end) from the other
            r.sc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 rs0, (int)(srow_up ? kPastEnd : sofs), 0, 0));
            r.sc2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                  rs1, (int)(srow_up ? sofs : kPastEnd), 0, 0));
        } else {
            r.sc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs0, (int)sofs, 0, 0));
        }
        if constexpr (!HOLD) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
                r.hid[b] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rx, (int)(xlane + (uint32_t)(blk0 + b) * kBlock * 2u), 0, 0));
        }
    };

    // ---- prologue ------------------------------------------------------------------------
    // Held rows: the window rows and the norm's sum-of-squares partials are issued first and
    // the ring after them, so the norm waits for its own loads only while the ring's are in
    // flight (issued the other way round, the norm's wait drained the whole ring).  The
    // partials are read with uniform buffer loads (zeros past the end, and everywhere when
    // there is no norm), each lane folding 4 consecutive partials, the order norm_scales uses.
    Unit<HOLD> ring[DEPTH];
    f16x8 hold[HOLD ? HOLD : 1][4];
    float inv = 1.0f;
    if constexpr (HOLD > 0) {
        constexpr int RPN = (16 + NW - 1) / NW;            // window rows whose norm this wave folds
#pragma unroll
        for (int c = 0; c < HOLD; ++c)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                hold[c][b] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rx, (int)(xlane + (uint32_t)(kbase + c * NW * 4 + wave * 4 + b) * kBlock * 2u),
                                                           0, 0));
        // H <= 4096 here (at most two chunks of 16 x 128 bytes), so nt = H / 16 <= 256: one
        // 4-wide load per lane and row covers all partials
        const int nt = a.norm_tiles;
        const __amdgpu_buffer_rsrc_t rn = buf_view(a.norm_ss, a.norm_ss ? (uint32_t)a.S * (uint32_t)nt * 4u : 0u);
        f32x4 pv[RPN];
#pragma unroll
        for (int j = 0; j < RPN; ++j) {
            const int s = wave + j * NW;
            const uint32_t off = s < 16 && s < a.S && 4 * lane < nt ? ((uint32_t)s * nt + 4u * lane) * 4u : kPastEnd;
            pv[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rn, (int)off, 0, 0));
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(ring[d], d / HOLD, d % HOLD);
#pragma unroll
        for (int j = 0; j < RPN; ++j) {
            const int s = wave + j * NW;
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) t += pv[j][e];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, kWave);
            if (lane == 0 && s < 16) inv_s[s] = 1.0f / sqrtf(t / (float)a.H + a.eps);
        }
        lds_sync();
        inv = a.norm_ss && row_ok ? inv_s[n] : 1.0f;
#pragma unroll
        for (int c = 0; c < HOLD; ++c)
#pragma unroll
            for (int b = 0; b < 4; ++b) hold[c][b] = a.norm_ss ? scale_f16x8(hold[c][b], inv) : hold[c][b];
    } else {
        // streamed rows: the ring first, then the norm (its loads are the youngest)
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(ring[d], 0, d);
        if (a.norm_ss) {
            norm_scales<NW>(a.norm_ss, a.norm_tiles, a.S, a.H, a.eps, wave, lane, inv_s);
            lds_sync();
            if (row_ok) inv = inv_s[n];
        }
    }

    // ---- distributed epilogue: wave w finishes window rows w, w + NW, ... of every tile --
    const uint32_t out_elems = (uint32_t)a.S * (uint32_t)a.V;
    const __amdgpu_buffer_rsrc_t ry = buf_view(a.y, a.y ? out_elems * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rres = buf_view(a.residual, a.residual ? out_elems * 2u : 0u);
    const __amdgpu_buffer_rsrc_t rlog = buf_view(a.logits, a.logits ? out_elems * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rss = buf_view(a.ss_out, a.ss_out ? (uint32_t)a.S * (uint32_t)a.nitems * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rkp = buf_view(a.kpart, ks > 1 ? (uint32_t)ks * out_elems * 4u : 0u);
    float best_v[RPW];
    int best_i[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) { best_v[j] = -INFINITY; best_i[j] = INT_MAX; }

    auto finish_tile = [&](const f32x4& acc, int k, int buf) {
        red[buf][wave][lane] = acc;
        lds_sync();
        const int it = first + k * step;
        const bool live = k < my_items;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int s = wave + j * NW;                       // window row (compile-time count)
            const int sr = s & 15;                             // rows >= 16 read a real slot, store nothing
            const float* col = reinterpret_cast<const float*>(&red[buf][0][n + 16 * (sr >> 2)]) + (sr & 3);
            float val = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) val += col[w * kWave * 4];
            const int v = crow<EPI>(it, n);
            const bool ok = live && lane < 16 && s < 16 && s < a.S && v < a.V;
            if constexpr (EPI == EPI_GATEUP) {
                const float up = __shfl_xor(val, 8, 16);
                const float out = val / (1.0f + expf(-val)) * up;
                const uint32_t off = ok && n < 8 ? ((uint32_t)s * a.V + v) * 2u : kPastEnd;
                __builtin_amdgcn_raw_buffer_store_b16(f2h(out), ry, (int)off, 0, 0);
            } else if constexpr (EPI == EPI_HEAD) {
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rlog,
                                                      (int)(ok ? ((uint32_t)s * a.V + v) * 4u : kPastEnd), 0, 0);
                if (ok && val > best_v[j]) { best_v[j] = val; best_i[j] = v; }
            } else if (ks > 1) {
                // this slice's share of the tile: the epilogue runs after the fold
                const uint32_t off = ok ? (((uint32_t)slice * a.S + s) * a.V + v) * 4u : kPastEnd;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rkp, (int)off, 0, kAuxDevice);
            } else {
                const uint32_t off = ok ? ((uint32_t)s * a.V + v) * 2u : kPastEnd;
                val += h2f(__builtin_amdgcn_raw_buffer_load_b16(rres, (int)off, 0, 0));    // zero without a residual
                const uint16_t hv = f2h(val);
                __builtin_amdgcn_raw_buffer_store_b16(hv, ry, (int)off, 0, 0);
                const float q = ok ? h2f(hv) : 0.f;
                float sq = q * q;
#pragma unroll
                for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 16);
                const bool first = ok && n == 0;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sq), rss,
                                                      (int)(first ? ((uint32_t)s * a.nitems + it) * 4u : kPastEnd), 0, 0);
            }
        }
    };

    // ---- consume one unit: LDS exchange into the MFMA layout, 4 blocks -------------------
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const Unit<HOLD>& cur, int slot, const f16x8 (&aops)[4], f32x4& acc) {
        uint8_t* xs = xch[wave][slot];
        // exchange: tile row r lands at r*128, 16-byte chunks XOR-swizzled by row
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 8 * h + lrow;
            *reinterpret_cast<u32x4*>(xs + row * 128 + 16 * (lchunk ^ (row & 7))) = cur.w[h];
        }
        // each block's scale is applied one block later (the last one after the loop), so no
        // instruction waits on a just-issued MFMA; the accumulation order is unchanged
        f32x4 dprev = zero;
        float scprev = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int chunk = 2 * b + (g >> 1);
            const u32x2 q8 = *reinterpret_cast<const u32x2*>(xs + n * 128 + 16 * (chunk ^ (n & 7)) + 8 * (g & 1));
            const f16x8 bop = i8x8_to_f16x8(q8);
            const u32x2 scw = EPI == EPI_GATEUP ? (cur.sc | cur.sc2) : cur.sc;
            const float sc = h2f((uint16_t)(scw[b >> 1] >> (16 * (b & 1))));
            const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(aops[b], bop, zero, 0, 0, 0);
            if (b > 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(scprev, dprev[r], acc[r]);
            }
            dprev = dd;
            scprev = sc;
            if constexpr (NW == 16) __builtin_amdgcn_sched_barrier(0);   // bound live temporaries at 16 waves
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(scprev, dprev[r], acc[r]);
    };

    if constexpr (HOLD > 0) {
        constexpr int TPC = DEPTH / HOLD;                // tiles per ring cycle
        const int ncycles = (my_items + TPC - 1) / TPC;
        for (int cy = 0; cy < ncycles; ++cy) {
            f32x4 acc = zero;
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int k = cy * TPC + d / HOLD;
                consume(ring[d], d & 1, hold[d % HOLD], acc);
                load(ring[d], k + TPC, d % HOLD);        // the same slot, one cycle ahead
                if (d % HOLD == HOLD - 1) {
                    finish_tile(acc, k, k & 1);
                    acc = zero;
                }
            }
        }
    } else {
        for (int k = 0; k < my_items; ++k) {
            f32x4 acc = zero;
            for (int c0 = 0; c0 < nkc; c0 += DEPTH) {
#pragma unroll
                for (int d = 0; d < DEPTH; ++d) {
                    f16x8 aops[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) aops[b] = a.norm_ss ? scale_f16x8(ring[d].hid[b], inv) : ring[d].hid[b];
                    consume(ring[d], d & 1, aops, acc);
                    const int c = c0 + d + DEPTH;         // the same slot, DEPTH units ahead
                    const bool next = c >= nkc;
                    load(ring[d], next ? k + 1 : k, next ? c - nkc : c);
                }
            }
            finish_tile(acc, k, k & 1);
        }
    }

    if constexpr (EPI == EPI_STORE) {
        if (ks > 1) {
            // Fold.  Every wave waits until its device-coherent share stores are acknowledged
            // (vector memory count zero), then one lane per tile of this workgroup counts the
            // tile's arrival with a device-scope atomic; the workgroup that brings a tile's
            // count to kslices is the last to have written its share, and it reads the kslices
            // shares with device-coherent loads, adds them in slice order (the same order
            // whichever workgroup folds) and runs the store epilogue: residual, fp16 store,
            // per-tile sum of squares in the butterfly order of the unsplit epilogue.  It
            // leaves the counter at zero for the next launch.
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (wave == 0) {
                const int it = first + lane * step;
                bool last = false;
                if (lane < my_items)
                    last = __hip_atomic_fetch_add(a.counters + it, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                           (uint32_t)(ks - 1);
                const uint64_t bal = __ballot(last);
                if (last) fold_it[__builtin_popcountll(bal & ((1ull << lane) - 1ull))] = it;
                if (lane == 0) fold_n = __builtin_popcountll(bal);
            }
            __syncthreads();
            const int nf = fold_n;
            if (nf > 0) {
                const int total = nf * a.S;
                // four (tile, window row) pairs per wave and pass, one tile row per lane
                for (int q0 = wave * 4; q0 < total; q0 += NW * 4) {
                    const int q = q0 + g;
                    const bool qok = q < total;
                    const int j = qok ? q / a.S : 0;
                    const int s = qok ? q - j * a.S : 0;
                    const int it = fold_it[j];
                    const int v = it * kTileRows + n;
                    const bool ok = qok && v < a.V;
                    float p[kMaxSlices];
#pragma unroll
                    for (int k = 0; k < kMaxSlices; ++k) {
                        const uint32_t off = ok && k < ks ? (((uint32_t)k * a.S + s) * a.V + v) * 4u : kPastEnd;
                        p[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rkp, (int)off, 0, kAuxDevice));
                    }
                    float val = p[0];
#pragma unroll
                    for (int k = 1; k < kMaxSlices; ++k)
                        if (k < ks) val += p[k];
                    const uint32_t off = ok ? ((uint32_t)s * a.V + v) * 2u : kPastEnd;
                    val += h2f(__builtin_amdgcn_raw_buffer_load_b16(rres, (int)off, 0, 0));
                    const uint16_t hv = f2h(val);
                    __builtin_amdgcn_raw_buffer_store_b16(hv, ry, (int)off, 0, 0);
                    const float qv = ok ? h2f(hv) : 0.f;
                    float sq = qv * qv;
#pragma unroll
                    for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 16);
                    const bool first_row = ok && n == 0;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sq), rss,
                                                          (int)(first_row ? ((uint32_t)s * a.nitems + it) * 4u : kPastEnd),
                                                          0, 0);
                    if (first_row && s == 0)
                        __hip_atomic_store(a.counters + it, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }

    if constexpr (EPI == EPI_HEAD) {
        const __amdgpu_buffer_rsrc_t rpv = buf_view(a.part_val, (uint32_t)a.S * kGridMax * 4u);
        const __amdgpu_buffer_rsrc_t rpi = buf_view(a.part_idx, (uint32_t)a.S * kGridMax * 4u);
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            float bv = best_v[j];
            int bi = best_i[j];
            argmax_group<16>(bv, bi);
            const int s = wave + j * NW;
            const uint32_t off = lane == 0 && s < 16 && s < a.S ? ((uint32_t)s * kGridMax + blockIdx.x) * 4u : kPastEnd;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, bv), rpv, (int)off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)bi, rpi, (int)off, 0, 0);
        }
    }
}

// ss[s][t] = sum over the 16 columns of tile t of fp16(x[s, k])^2: the partials of a stream
// that did not come out of a down projection (the stack's input).  The square of an fp16
// value is exact in fp32, and the 16 squares are added in the order of the down epilogue's
// butterfly (columns k and k+8, then +4, +2, +1), so a stream gets the same partials here as
// from a down projection that stored it: a block computes the same bits whether its input
// came from the previous block of one call or from the caller.
__global__ __launch_bounds__(256) void row_ss_kernel(const uint16_t* __restrict__ x, int S, int H,
                                                     float* __restrict__ ss, uint32_t* __restrict__ zero, int nzero) {
    const int nt = H / kTileRows;
    const int s = blockIdx.y;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (s == 0)
        for (int i = t; i < nzero; i += gridDim.x * 256) zero[i] = 0u;
    if (s >= S || t >= nt) return;
    const uint16_t* p = x + (size_t)s * H + (size_t)t * kTileRows;
    float sq[kTileRows];
#pragma unroll
    for (int k = 0; k < kTileRows; ++k) {
        const float q = h2f(p[k]);
        sq[k] = q * q;
    }
#pragma unroll
    for (int w = kTileRows / 2; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) sq[k] = sq[k] + sq[k + w];
    ss[(size_t)s * nt + t] = sq[0];
}

// out[s, k] = fp16(x[s, k] * inv[s]) with inv from the ss partials exactly as the gate/up
// prologue computes it.  One workgroup per window row.
__global__ __launch_bounds__(256) void apply_norm_kernel(const uint16_t* __restrict__ x, const float* __restrict__ ss,
                                                         int S, int H, float eps, uint16_t* __restrict__ out) {
    __shared__ float inv_s[kTileRows];
    const int s = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the same fixed summation order as the gate/up prologue (norm_scales), for row s only
    if (wave == 0) norm_scales<1>(ss + (size_t)s * (H / kTileRows), H / kTileRows, 1, H, eps, 0, lane, inv_s);
    __syncthreads();
    const float inv = inv_s[0];
    for (int k = threadIdx.x; k < H; k += 256) out[(size_t)s * H + k] = f2h(h2f(x[(size_t)s * H + k]) * inv);
}

typedef void (*ChunkFn)(ChunkArgs);

// (waves, hold, depth) -> kernel; hold = 0 streams the window rows with each unit.  Only
// shapes that compile without register spills on gfx950 are instantiated.
template <int EPI>
ChunkFn pick_chunked(int nw, int hold, int depth) {
#define SV_CH(NW, HOLD, DEPTH) \
    if (nw == NW && hold == HOLD && depth == DEPTH) return q8b32_chunked<NW, DEPTH, HOLD, EPI>;
    SV_CH(16, 0, 2) SV_CH(16, 1, 2) SV_CH(16, 1, 4) SV_CH(16, 2, 2)
    SV_CH(14, 0, 2) SV_CH(14, 1, 2) SV_CH(14, 2, 2)
    SV_CH(12, 0, 2) SV_CH(12, 0, 3) SV_CH(12, 1, 2) SV_CH(12, 1, 4) SV_CH(12, 2, 2) SV_CH(12, 2, 4)
    SV_CH(10, 0, 2) SV_CH(10, 1, 2) SV_CH(10, 2, 2)
    SV_CH(8, 0, 2) SV_CH(8, 0, 3) SV_CH(8, 0, 4) SV_CH(8, 1, 2) SV_CH(8, 1, 4) SV_CH(8, 2, 2) SV_CH(8, 2, 4)
    SV_CH(4, 0, 2) SV_CH(4, 0, 3) SV_CH(4, 0, 4) SV_CH(4, 1, 4) SV_CH(4, 2, 4)
#undef SV_CH
    return nullptr;
}

ChunkFn chunked_fn(int epi, int nw, int hold, int depth) {
    if (epi == EPI_HEAD) return pick_chunked<EPI_HEAD>(nw, hold, depth);
    if (epi == EPI_STORE) return pick_chunked<EPI_STORE>(nw, hold, depth);
    return pick_chunked<EPI_GATEUP>(nw, hold, depth);
}

int device_cus() {
    static int cache[64] = {0};
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev]) return cache[dev];
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        return 256;
    }
    cache[dev] = cus;       // a benign race: every thread writes the same value
    return cus;
}

int chunked_resident(ChunkFn fn, int nw) {
    struct Entry { ChunkFn fn; int dev; int groups; };
    static Entry cache[32];
    static int used = 0;
    static std::mutex mu;
    int dev = -1;
    const int fallback = nw >= 16 ? 256 : 512;
    if (hipGetDevice(&dev) != hipSuccess) return fallback;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].groups;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), nw * 64, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1) {
        (void)hipGetLastError();
        return fallback;
    }
    if (used < 32) cache[used++] = Entry{fn, dev, per_cu * cus};
    return per_cu * cus;
}

}  // namespace

namespace {
thread_local int g_chunk_nw = 0;       // tuning overrides of the calling thread, 0 = automatic
thread_local int g_chunk_depth = 0;
thread_local int g_grid_override_chunk = 0;
thread_local int g_head_kernel = 0;    // 0 automatic, 1 one-pass-per-item kernel, 2 ring kernel
thread_local int g_down_split = 0;     // 0 or 1 unsplit, k > 1 k slices when possible
}  // namespace

void set_chunk_tuning(int waves, int depth, int max_groups, int head_kernel, int split) {
    g_chunk_nw = waves;
    g_chunk_depth = depth;
    g_grid_override_chunk = max_groups;
    g_head_kernel = head_kernel;
    g_down_split = split;
}

bool head_use_chunked(int V, int H) {
    (void)V;
    (void)H;
    return g_head_kernel == 2;
}

namespace {

// Held-row shape of one slice of Hs hidden columns: Hs = hold x nw x 128 bytes, hold <= 2, the
// deepest ring that compiles without spills.
bool slice_shape(int epi, int Hs, int& nw_out, int& hold_out, int& depth_out) {
    if (Hs % 128) return false;
    const int segs = Hs / 128;
    for (int nw : {16, 12, 8, 14, 10, 4})
        for (int hold : {1, 2}) {
            if (segs != nw * hold || (g_chunk_nw && nw != g_chunk_nw)) continue;
            int depth = 0;
            for (int d : {4, 3, 2})
                if (!depth && chunked_fn(epi, nw, hold, d)) depth = d;
            if (g_chunk_depth && chunked_fn(epi, nw, hold, g_chunk_depth)) depth = g_chunk_depth;
            if (!depth) continue;
            nw_out = nw;
            hold_out = hold;
            depth_out = depth;
            return true;
        }
    return false;
}

// A store projection's hidden axis split ks ways: one workgroup per compute unit at most,
// kslices x gps workgroups, each taking one slice (its window rows held in registers) and
// ceil(tiles / gps) tiles.
bool split_config(int rows, int H, int ks, ChunkCfg& c) {
    if (ks < 2 || ks > kMaxSlices || H % ks) return false;
    int nw, hold, depth;
    if (!slice_shape(EPI_STORE, H / ks, nw, hold, depth)) return false;
    const int tiles = (rows + kTileRows - 1) / kTileRows;
    int cap = device_cus();
    if (g_grid_override_chunk > 0 && g_grid_override_chunk < cap) cap = g_grid_override_chunk;
    int gps = cap / ks;
    if (gps < 1) return false;
    const int per = (tiles + gps - 1) / gps;
    if (per > kMaxSliceItems) return false;
    gps = (tiles + per - 1) / per;
    c.nw = nw;
    c.nkc = hold;
    c.hold = hold;
    c.depth = depth;
    c.grid = gps * ks;
    c.items = tiles;
    c.ks = ks;
    return true;
}

}  // namespace

size_t chunked_split_bytes(int rows, int H, int S) {
    ChunkCfg c;
    if (!chunked_config(rows, H, EPI_STORE, c, S) || c.ks < 2) return 0;
    const size_t part = ((size_t)4 * c.ks * S * rows + 255) & ~(size_t)255;
    return part + (((size_t)4 * c.items + 255) & ~(size_t)255);
}

bool chunked_config(int rows, int H, int epi, ChunkCfg& c, int S) {
    const int nb = H / kBlock;
    if (H % kBlock || nb % 4) return false;
    if ((uint64_t)rows * (uint64_t)H >= (1ull << 31)) return false;     // 32-bit buffer offsets
    c.ks = 1;
    const int segs = nb / 4;
    // measured preference: the streamed-row down projection is fastest at 8 waves, the
    // held-row shapes at 16
    const int pref[2][6] = {{16, 14, 12, 10, 8, 4}, {8, 16, 14, 12, 10, 4}};
    for (int nw : pref[epi == EPI_STORE ? 1 : 0]) {
        if (segs % nw) continue;
        if (g_chunk_nw && nw != g_chunk_nw) continue;
        c.nw = nw;
        c.nkc = segs / nw;
        c.hold = c.nkc <= 2 ? c.nkc : 0;
        // deepest ring that compiles without spills at this width (see pick_chunked)
        // held rows: the deepest ring that compiles without spills; streamed rows: the
        // shallowest ring that divides the chunks (measured: deeper rings hold more window-row
        // registers than they gain)
        auto fits = [&](int d) { return chunked_fn(epi, nw, c.hold, d) && (c.hold || c.nkc % d == 0); };
        int depth = 0;
        if (c.hold) {
            for (int d : {4, 3, 2})
                if (!depth && fits(d)) depth = d;
        } else {
            for (int d : {2, 3, 4})
                if (!depth && fits(d)) depth = d;
        }
        if (g_chunk_depth && fits(g_chunk_depth)) depth = g_chunk_depth;       // else automatic
        if (!depth) continue;
        c.depth = depth;
        const int items = epi == EPI_GATEUP ? (rows + 7) / 8 : (rows + kTileRows - 1) / kTileRows;
        int cap = chunked_resident(chunked_fn(epi, nw, c.hold, depth), nw);
        if (g_grid_override_chunk > 0) cap = g_grid_override_chunk;
        if (cap > kGridMax) cap = kGridMax;
        const int per = (items + cap - 1) / cap;
        c.grid = (items + per - 1) / per;
        c.items = items;
        if (epi == EPI_STORE && S > 0 && g_down_split > 1) {
            // Taken only when the calling thread asks for it.  Measured on the dense-stack
            // block (4096 rows, 12288 columns, S = 9): the split streams 40-45% fewer bytes
            // per workgroup, yet its launch is not shorter (17.8 us at 4 slices, 20.9 us at 8,
            // against 17.0 us unsplit): a held window slice must arrive before the first
            // product, and it queues behind the whole ring burst at launch (about 6 us),
            // while the unsplit kernel's first unit brings its own window rows.
            ChunkCfg sc;
            if (split_config(rows, H, g_down_split, sc)) c = sc;
        }
        return true;
    }
    return false;
}

hipError_t launch_chunked(int epi, const ChunkCfg& c, const ChunkArgs& a, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    ChunkFn fn = chunked_fn(epi, c.nw, c.hold, c.depth);
    if (!fn) return hipErrorInvalidConfiguration;
    launch_timed(fn, dim3(c.grid), dim3(c.nw * 64), stream, start, stop, a);
    return hipGetLastError();
}

hipError_t launch_row_ss(const uint16_t* x, int S, int H, float* ss, uint32_t* zero, int nzero,
                         hipStream_t stream) {
    const int nt = H / kTileRows;
    hipLaunchKernelGGL(row_ss_kernel, dim3((nt + 255) / 256, S), dim3(256), 0, stream, x, S, H, ss, zero, nzero);
    return hipGetLastError();
}

hipError_t launch_apply_norm(const uint16_t* x, const float* ss, int S, int H, float eps, uint16_t* out,
                             hipStream_t stream) {
    hipLaunchKernelGGL(apply_norm_kernel, dim3(S), dim3(256), 0, stream, x, ss, S, H, eps, out);
    return hipGetLastError();
}

}  // namespace sv
