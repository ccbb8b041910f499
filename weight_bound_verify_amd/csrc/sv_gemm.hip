// q8b32 skinny matmul for gfx950: int8 rows with per-block-32 fp16 scales against S <= 64
// fp16 activation rows, fp32 accumulation, one pass over the weights (two for an argmax head
// of more than 32 window rows, where head_config runs the two-tile kernel twice).
//
// Contraction (pages: "Riding Apple's pipelined GPU engine", quantization on the GPU
// delegate -- linear per-block-32 int8; "Stream C - Speculative decoding", C1 substrate map
// and the delta -- all-position logits of the S = K+1 window, batched per-row argmax):
//   L[s, v] = sum_b f32(scale[v, b]) * sum_{k in block b} f32(q[v, k]) * f32(x[s, k])
//
// Mapping onto v_mfma_f32_16x16x32_f16 (one instruction = one 32-wide quantization block):
//   B operand (32 x 16) = the block of 16 weight rows; lane l holds row l%16, codes
//                         8*(l/16) .. +7 of the block, converted exactly to fp16.
//   A operand (16 x 32) = the matching block of 16 window rows (zeros past S), held in
//                         registers for the whole launch.
//   D (16 x 16) fp32    = lane l holds window rows 4*(l/16) .. +3 of weight row l%16, so the
//                         block scale of that weight row multiplies all four in fp32:
//                         acc += scale * D.  Every product (an integer code times an fp16
//                         value) is exact in fp32; the sums, within a block and across blocks,
//                         round in fp32.
// A workgroup owns 16 weight rows at a time ("item"); its NW waves split the hidden axis,
// each holding its share of the window rows in registers, and reduce through LDS in a fixed
// order (deterministic).  The head epilogue keeps a running (value, lowest index) argmax
// per window row; only 8 bytes per (window row, workgroup) leave the kernel.  The next
// item's loads are issued before the current item's math (two alternating register sets).
//
// Two kernels share this structure:
//   q8b32_fast     each load instruction reads 8 rows x 128 contiguous bytes (the access
//                  pattern that streams HBM near its peak; 16 rows x 8 bytes per
//                  instruction, the MFMA operand layout, streams at about half of it).  Each
//                  wave exchanges the bytes into the MFMA layout through two 2 KB LDS slots
//                  of its own, XOR-swizzled by row so both the 16-byte writes and the 8-byte
//                  reads are free of bank conflicts.  Every wave's share of the hidden axis
//                  must be a whole number of 128-byte segments.
//   q8b32_generic  any shape: each lane loads its 8 MFMA bytes directly.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_tail.h"

#include <climits>
#include <cmath>
#include <mutex>

namespace sv {

namespace {

thread_local int g_nw_override = 0;       // tuning overrides of the calling thread, 0 = choose
thread_local int g_grid_override = 0;     // 0 = choose
thread_local int g_no_xr = 0;            // 1: a 17-row window uses the two-tile kernels (tuning experiments)

constexpr int kXcds = 8;         // accelerator dies; workgroup b of a launch runs on die b % kXcds

// The items a workgroup of a persistent grid takes: first, first + step, ... below lim.  By
// default workgroup b takes b, b + grid, ...  With `xcd` the items split into kXcds contiguous
// ranges, one per die, and the workgroups of a die stride through its range (taken only when
// every workgroup then has an item: at least kXcds workgroups and kXcds items per workgroup).
// Either order covers every item exactly once, so results never depend on where the hardware
// actually places the workgroups; only the speed does.
struct ItemRange {
    int first, step, lim;
};
__device__ __forceinline__ ItemRange item_range(int nitems, bool xcd) {
    const int b = blockIdx.x, grid = gridDim.x;
    if (xcd && grid >= kXcds && nitems >= kXcds * grid) {
        const int x = b % kXcds;
        return {(int)((long long)nitems * x / kXcds) + b / kXcds, (grid - x + kXcds - 1) / kXcds,
                (int)((long long)nitems * (x + 1) / kXcds)};
    }
    return {b, grid, nitems};
}

// Workgroup barrier that orders LDS only, so prefetched global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Window rows for blocks [bw0, bw0 + nbw) in this lane's A-operand slots.
template <int MT, int NBW>
__device__ __forceinline__ void load_hidden(f16x8 (&hid)[NBW][MT], const GemmArgs& a, int bw0, int nbw, int n,
                                            int g) {
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int s = mt * 16 + n;
            f16x8 h = {};
            if (i < nbw && s < a.S)
                h = *reinterpret_cast<const f16x8*>(a.x + (size_t)s * a.H + (size_t)(bw0 + i) * kBlock + g * 8);
            hid[i][mt] = h;
        }
    }
}

// Weight row feeding MFMA tile row n (0..15) of item `it`.  Head and plain projections: 16
// rows of one matrix.  Gate/up: tile rows 0..7 are 8 rows of the gate matrix and 8..15 the
// same 8 rows of the up matrix, so one tile yields both operands of silu(g) * u and the two
// 8-row halves of a tile map onto the two 8-row load instructions of the fast kernel.
template <int EPI>
__device__ __forceinline__ int tile_row(int it, int n) {
    return EPI == EPI_GATEUP ? it * 8 + (n & 7) : it * kTileRows + n;
}
template <int EPI>
__device__ __forceinline__ bool tile_up(int n) { return EPI == EPI_GATEUP && n >= 8; }

// Cross-wave reduction of one item through LDS, then the epilogue in wave 0.
template <int MT, int NW, int EPI>
struct Reducer {
    f32x4 (*red)[NW][MT][kWave];
    float best_v[MT][4];
    int best_i[MT][4];
    // EPI_SAMPLE (MT = 1): running max of z and sum of exp(z - max) per window row of the
    // lane, the draft each row leaves out of its draw, the round's start position, and three
    // LDS slots of Gumbel noise [lane] (rows 4g..4g+3 of id n of an item), filled one item
    // ahead by a wave other than wave 0 so the generator stays off the epilogue's path
    float run_m[4], run_l[4];
    int excl[4];
    uint32_t p0;
    f32x4 (*noise)[kWave];
    int kloc;                  // items this workgroup has processed

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) { best_v[mt][r] = -INFINITY; best_i[mt][r] = INT_MAX; }
#pragma unroll
        for (int r = 0; r < 4; ++r) { run_m[r] = -INFINITY; run_l[r] = 0.0f; excl[r] = -1; }
        p0 = 0;
        kloc = 0;
    }

    // Per-round inputs of the sampling epilogue (every wave: the start position; wave 0: the
    // drafts it leaves out), then the noise of the workgroup's first item.
    __device__ __forceinline__ void setup(const GemmArgs& a, int wave, int lane, int first) {
        if constexpr (EPI == EPI_SAMPLE) {
            const int g = lane >> 4;
            p0 = (uint32_t)a.state[SV_STATE_LEN];
            if (wave == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 4 * g + r;
                    excl[r] = s < a.S - 1 ? a.drafts[s] : -1;
                }
            }
            if (wave == (NW > 1 ? 1 : 0)) make_noise(a, first, 0, lane);
        }
    }

    // Gumbel noise of item `item` into slot `slot`: lane (n, g) draws rows 4g..4g+3 of id
    // 16 item + n from one Philox block (counter (v, P0, g, 0)).
    __device__ __forceinline__ void make_noise(const GemmArgs& a, int item, int slot, int lane) {
        const int n = lane & 15, g = lane >> 4;
        const int v = item * kTileRows + n;
        f32x4 out = {0.f, 0.f, 0.f, 0.f};
        if (item < a.nitems && 4 * g < a.S && v < a.V) {
            const Philox4 rnd = philox4x32_10((uint32_t)v, p0, (uint32_t)g, 0u, a.key0, a.key1);
#pragma unroll
            for (int r = 0; r < 4; ++r) out[r] = gumbel(uniform01(rnd.w[r]));
        }
        noise[slot][lane] = out;
    }

    // Called at the start of each item by every wave: the item after this one gets its noise
    // from wave 1 + (k mod (NW - 1)) while that wave's loads are in flight.  Slots rotate
    // over three items, so the slot written (k + 1) was last read by wave 0 in the epilogue of
    // item k - 2, which ended before that wave passed the barrier of item k - 1.
    __device__ __forceinline__ void ahead(const GemmArgs& a, int next_item, int wave, int lane) {
        if constexpr (EPI == EPI_SAMPLE) {
            if (a.ksplit == 1) {
                const int writer = NW > 1 ? 1 + kloc % (NW - 1) : 0;
                if (wave == writer) make_noise(a, next_item, (kloc + 1) % 3, lane);
            }
        }
    }

    __device__ __forceinline__ void run(const GemmArgs& a, const f32x4 (&acc)[MT], int it, int buf, int wave, int lane,
                                        int ks) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[buf][wave][mt][lane] = acc[mt];
        lds_barrier();
        const int kcur = kloc;
        kloc = kcur + 1;
        if (wave != 0) return;

        f32x4 tot[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 t = red[buf][0][mt][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) t += red[buf][w][mt][lane];
            tot[mt] = t;
        }
        const int n = lane & 15, g = lane >> 4;
        const int v = tile_row<EPI>(it, n);
        if constexpr (EPI == EPI_SAMPLE) {
            // z = L / T; key = z + Gumbel noise of (row, id) with the row's draft left out;
            // online log-sum-exp of z.  Ids arrive in increasing order, so a strict > keeps
            // the lowest id on equal keys.
            if (a.ksplit == 1 && 4 * g < a.S && v < a.V) {
                const f32x4 gn = noise[kcur % 3][lane];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 4 * g + r;
                    if (s < a.S) {
                        const float L = tot[0][r];
                        if (a.logits) a.logits[(size_t)s * a.V + v] = L;
                        const float z = L * a.inv_temp;
                        const bool out = v == excl[r];
                        if (out) a.zd[s] = z;
                        const float key = out ? -INFINITY : z + gn[r];
                        if (key > best_v[0][r]) { best_v[0][r] = key; best_i[0][r] = v; }
                        if (z > run_m[r]) {
                            run_l[r] = run_l[r] * __expf(run_m[r] - z) + 1.0f;
                            run_m[r] = z;
                        } else {
                            run_l[r] += __expf(z - run_m[r]);
                        }
                    }
                }
            } else if (a.ksplit > 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = g * 4 + r;
                    if (s < a.S && v < a.V) a.kpart0[(size_t)ks * a.S * a.V + (size_t)s * a.V + v] = tot[0][r];
                }
            }
            return;
        }
        if constexpr (EPI == EPI_GATEUP) {
            // lanes n < 8 hold the gate sums, lanes n + 8 the up sums of the same output rows
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float other = __shfl_xor(tot[mt][r], 8, 16);
                    const int s = mt * 16 + g * 4 + r;
                    if (s < a.S && v < a.V) {
                        const size_t o = (size_t)s * a.V + v;
                        if (a.ksplit > 1) {
                            float* part = n < 8 ? a.kpart0 : a.kpart1;
                            part[(size_t)ks * a.S * a.V + o] = tot[mt][r];
                        } else if (n < 8) {
                            const float gg = tot[mt][r];
                            a.y[o] = f2h(gg / (1.0f + expf(-gg)) * other);
                        }
                    }
                }
            return;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = mt * 16 + g * 4 + r;
                if (s < a.S && v < a.V) {
                    const size_t o = (size_t)s * a.V + v;
                    if (a.ksplit > 1) {
                        a.kpart0[(size_t)ks * a.S * a.V + o] = tot[mt][r];
                    } else if constexpr (EPI == EPI_HEAD) {
                        const float val = tot[mt][r];
                        if (a.logits) a.logits[o] = val;
                        if (val > best_v[mt][r]) { best_v[mt][r] = val; best_i[mt][r] = v; }
                    } else {
                        float val = tot[mt][r];
                        if (a.residual) val += h2f(a.residual[o]);
                        a.y[o] = f2h(val);
                    }
                }
            }
    }

    // Per-workgroup argmax partials of the head (wave 0); for sampling also the per-row
    // (max, sum of exp) pairs, merged across the 16 lanes of a row in a fixed order.
    __device__ __forceinline__ void finish(const GemmArgs& a, int lane) {
        const int n = lane & 15, g = lane >> 4;
        if constexpr (EPI == EPI_SAMPLE) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m = run_m[r], l = run_l[r];
                lse_merge_group<16>(m, l);
                const int s = g * 4 + r;
                if (n == 0 && s < a.S) {
                    a.part_m[(size_t)s * kGridMax + blockIdx.x] = m;
                    a.part_l[(size_t)s * kGridMax + blockIdx.x] = l;
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float bv = best_v[mt][r];
                int bi = best_i[mt][r];
                argmax_group<16>(bv, bi);
                const int s = mt * 16 + g * 4 + r;
                if (n == 0 && s < a.S) {
                    a.part_val[(size_t)s * kGridMax + blockIdx.x] = bv;
                    a.part_idx[(size_t)s * kGridMax + blockIdx.x] = bi;
                }
            }
    }
};

// ------------------------------------------------------------------------------------------
// fast kernel
// ------------------------------------------------------------------------------------------
template <int NBW>
struct FastRegs {
    static constexpr int NSEG = NBW / 4;          // 128-byte segments per row per wave
    u32x4 w[NSEG][2];                              // [segment][row half]
    uint32_t sc[NBW / 2];                          // fp16 scales of the lane's row, in pairs
};

// XR > 0 (head, MT = 1; instantiated for XR = 1): window rows 16 .. 16+XR-1 beyond the MFMA tile.  Each wave keeps its
// blocks of them in LDS; per block a second MFMA takes the extra row, read from LDS as a
// broadcast, as all 16 of its A rows against the same codes, so each lane receives the row's
// full dot product with its vocab row, and adds it times the block scale.  A window of
// 17 .. 16+XR rows then needs the registers of a 16-row one and no split of the hidden axis.
// The waves' partials are folded in a fixed order by wave 1 + r for extra row r, which also
// keeps that row's running argmax.
//
// HL > 0 (MT = 1): the window rows of each wave's last HL blocks sit in LDS instead of
// registers (one 16-byte LDS read per block per lane), freeing 4 registers per block for shapes
// that would otherwise spill.
//
// ROLL = 1: one register set instead of two.  Each 128-byte segment of the next item is loaded
// into the registers of the same segment of the current item as soon as those have been
// written to the LDS exchange, and the next item's scales after the current item's last block,
// so one item's loads are in flight during the math as with two sets, in about half the
// registers.
template <int MT, int NBW, int NW, int EPI, int XR = 0, int HL = 0, int ROLL = 0>
__global__ __launch_bounds__(NW * 64) void q8b32_fast(GemmArgs a) {
    constexpr int NSEG = NBW / 4;
    constexpr int HR = NBW - HL;                      // blocks whose window rows stay in registers
    static_assert(NBW % 4 == 0, "whole 128-byte segments");
    static_assert(XR == 0 || (MT == 1 && EPI == EPI_HEAD && XR < NW), "extra rows extend a one-tile head");
    static_assert(HL == 0 || (MT == 1 && HL < NBW), "LDS-held blocks of a one-tile window");
    __shared__ f32x4 red[2][NW][MT][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xch[NW][2][2048];
    __shared__ f32x4 noise[EPI == EPI_SAMPLE ? 3 : 1][kWave];
    __shared__ __attribute__((aligned(16))) _Float16 xl[XR ? NW : 1][XR ? NBW : 1][XR ? XR : 1][kBlock];
    __shared__ float xred[XR ? 2 : 1][XR ? NW : 1][XR ? XR : 1][kTileRows];
    __shared__ __attribute__((aligned(16))) _Float16 xh[HL ? NW : 1][HL ? HL : 1][HL ? kTileRows : 1][kBlock];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int ks = blockIdx.y;
    const int bw0 = (a.nb / a.ksplit) * ks + NBW * wave;     // every wave owns exactly NBW blocks

    f16x8 hid[HR][MT];
    load_hidden<MT, HR>(hid, a, bw0, HR, n, g);
    if constexpr (HL > 0) {
        // rows 0..15 of this wave's last HL blocks, 16 bytes per lane per step; rows >= S are zeros
        for (int c = lane; c < HL * kTileRows * 4; c += kWave) {
            const int j = c / (kTileRows * 4), r = (c / 4) % kTileRows, q = c % 4;
            f16x8 v = {};
            if (r < a.S)
                v = *reinterpret_cast<const f16x8*>(a.x + (size_t)r * a.H + (size_t)(bw0 + HR + j) * kBlock + 8 * q);
            *reinterpret_cast<f16x8*>(&xh[wave][j][r][8 * q]) = v;
        }
    }
    float xbest_v = -INFINITY;          // extra row (wave - 1), lanes 0..15: running argmax
    int xbest_i = INT_MAX;
    if constexpr (XR > 0) {
        // rows 16 .. 16+XR-1 of this wave's blocks, 16 bytes per lane per step; rows >= S are zeros
        for (int c = lane; c < NBW * XR * 4; c += kWave) {
            const int i = c / (XR * 4), r = (c / 4) % XR, q = c % 4;
            f16x8 v = {};
            if (16 + r < a.S)
                v = *reinterpret_cast<const f16x8*>(a.x + (size_t)(16 + r) * a.H + (size_t)(bw0 + i) * kBlock + 8 * q);
            *reinterpret_cast<f16x8*>(&xl[wave][i][r][8 * q]) = v;
        }
    }

    Reducer<MT, NW, EPI> red_{red};
    red_.init();
    red_.noise = noise;
    // per-die item ranges for the argmax head only, and not for its shapes that hold window rows
    // in LDS (H = 5120, never given xcd); the others keep b, b + grid, ...
    ItemRange ir{(int)blockIdx.x, (int)gridDim.x, a.nitems};
    if constexpr (EPI == EPI_HEAD && HL == 0) ir = item_range(a.nitems, a.xcd != 0);
    red_.setup(a, wave, lane, ir.first);

    // loads: row half h feeds tile rows 8h .. 8h+7; lane l reads the tile row 8h + l/8, bytes
    // 16*(l%8) .. +15 of each 128-byte segment of the wave's range
    const int lrow = lane >> 3, lchunk = lane & 7;
    // segment t of an item's rows (both row halves)
    auto load_seg = [&](FastRegs<NBW>& r, int item, int t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int8_t* w = tile_up<EPI>(8 * h) ? a.w1 : a.w0;
            const int row = min(tile_row<EPI>(item, 8 * h + lrow), a.V - 1);      // tail rows: masked later
            const int8_t* p = w + (size_t)row * a.H + (size_t)bw0 * kBlock + 16 * lchunk;
            r.w[t][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 128 * t));
        }
    };
    auto load_sc = [&](FastRegs<NBW>& r, int item) {
        const uint16_t* s = tile_up<EPI>(n) ? a.s1 : a.s0;
        const int srow = min(tile_row<EPI>(item, n), a.V - 1);
        const uint16_t* sp = s + (size_t)srow * a.nb + bw0;
        if constexpr (NBW % 8 == 0) {
#pragma unroll
            for (int v = 0; v < NBW / 8; ++v) {
                const u32x4 q = *reinterpret_cast<const u32x4*>(sp + 8 * v);
#pragma unroll
                for (int e = 0; e < 4; ++e) r.sc[4 * v + e] = q[e];
            }
        } else {
#pragma unroll
            for (int v = 0; v < NBW / 4; ++v) {
                const u32x2 q = *reinterpret_cast<const u32x2*>(sp + 4 * v);
                r.sc[2 * v] = q.x;
                r.sc[2 * v + 1] = q.y;
            }
        }
    };
    auto load = [&](FastRegs<NBW>& r, int item) {
#pragma unroll
        for (int t = 0; t < NSEG; ++t) load_seg(r, item, t);
        load_sc(r, item);
    };

    // nxt: the item whose loads replace cur's registers as they free up (ROLL only)
    auto process = [&](FastRegs<NBW>& cur, int it, int buf, int nxt) {
        red_.ahead(a, it + ir.step, wave, lane);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = zero;
        float xacc[XR ? XR : 1];
#pragma unroll
        for (int r = 0; r < (XR ? XR : 1); ++r) xacc[r] = 0.f;
        // without extra rows each block's scale is applied one block later, so no instruction
        // waits on a just-issued MFMA (the accumulation order is unchanged); with them the extra
        // row's MFMA already fills that gap, and the delay measured slower
        constexpr bool kDelay = XR == 0;
        f32x4 dprev[MT];
        float scprev = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) dprev[mt] = zero;
#pragma unroll
        for (int t = 0; t < NSEG; ++t) {
            // exchange one segment: tile row r lands at r*128, 16-byte chunks XOR-swizzled by row
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 8 * h + lrow;
                *reinterpret_cast<u32x4*>(&xch[wave][t & 1][row * 128 + 16 * (lchunk ^ (row & 7))]) = cur.w[t][h];
            }
            if constexpr (ROLL) load_seg(cur, nxt, t);
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int i = 4 * t + bb;
                const int chunk = 2 * bb + (g >> 1);
                const int off = n * 128 + 16 * (chunk ^ (n & 7)) + 8 * (g & 1);
                const u32x2 q8 = *reinterpret_cast<const u32x2*>(&xch[wave][t & 1][off]);
                const f16x8 b = i8x8_to_f16x8(q8);
                const float sc = h2f((uint16_t)(cur.sc[i >> 1] >> (16 * (i & 1))));
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f16x8 aop = i < HR ? hid[i < HR ? i : 0][mt]
                                             : *reinterpret_cast<const f16x8*>(&xh[wave][i >= HR ? i - HR : 0][n][8 * g]);
                    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, b, zero, 0, 0, 0);
                    if constexpr (kDelay) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(scprev, dprev[mt][r], acc[mt][r]);
                        dprev[mt] = d;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(sc, d[r], acc[mt][r]);
                    }
                }
                if constexpr (XR > 0) {
#pragma unroll
                    for (int r = 0; r < XR; ++r) {
                        // extra row r repeated on all 16 A rows: every output row of this MFMA is
                        // its full 32-element dot with vocab row n, summed over the k groups
                        const f16x8 xv = *reinterpret_cast<const f16x8*>(&xl[wave][i][r][8 * g]);
                        const f32x4 d2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, b, zero, 0, 0, 0);
                        xacc[r] = __builtin_fmaf(sc, d2[0], xacc[r]);
                    }
                    if constexpr (NBW >= 16) __builtin_amdgcn_sched_barrier(0);   // bound live temporaries
                }
                scprev = sc;
            }
        }
        if constexpr (kDelay) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(scprev, dprev[mt][r], acc[mt][r]);
        }
        if constexpr (ROLL) load_sc(cur, nxt);
        if constexpr (XR > 0) {
            // the MFMA already summed the k groups: lanes n of group 0 hand the wave's partial
            // to LDS; the item's barrier in red_.run orders it before the readers
#pragma unroll
            for (int r = 0; r < XR; ++r)
                if (g == 0) xred[buf][wave][r][n] = xacc[r];
        }
        red_.run(a, acc, it, buf, wave, lane, ks);
        if constexpr (XR > 0) {
            const int r = wave - 1;                       // extra row handled by this wave
            if (r >= 0 && r < XR && 16 + r < a.S) {
                float val = xred[buf][0][r][n];
#pragma unroll
                for (int w = 1; w < NW; ++w) val += xred[buf][w][r][n];
                const int v = it * kTileRows + n;
                if (lane < 16 && v < a.V) {
                    if (a.logits) a.logits[(size_t)(16 + r) * a.V + v] = val;
                    if (val > xbest_v) { xbest_v = val; xbest_i = v; }
                }
            }
        }
    };

    const int step = ir.step, lim = ir.lim;
    const int last = lim - 1;
    int it = ir.first;
    if constexpr (ROLL) {
        FastRegs<NBW> r;
        load(r, min(it, last));
        for (int k = 0; it < lim; ++k, it += step) process(r, it, k & 1, min(it + step, last));
    } else {
        FastRegs<NBW> ra, rb;
        load(ra, it);
        while (true) {
            if (it >= lim) break;
            load(rb, min(it + step, last));
            process(ra, it, 0, 0);
            it += step;
            if (it >= lim) break;
            load(ra, min(it + step, last));
            process(rb, it, 1, 0);
            it += step;
        }
    }
    if constexpr (EPI == EPI_HEAD || EPI == EPI_SAMPLE)
        if (a.ksplit == 1 && wave == 0) red_.finish(a, lane);
    if constexpr (XR > 0) {
        const int r = wave - 1;
        if (r >= 0 && r < XR && 16 + r < a.S) {
            argmax_group<16>(xbest_v, xbest_i);
            if (lane == 0) {
                a.part_val[(size_t)(16 + r) * kGridMax + blockIdx.x] = xbest_v;
                a.part_idx[(size_t)(16 + r) * kGridMax + blockIdx.x] = xbest_i;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// generic kernel (any H; per-wave block counts may differ by one)
// ------------------------------------------------------------------------------------------
template <int NBW>
struct GenRegs {
    u32x2 w[NBW];
    uint16_t sc[NBW];
};

// Branch-free loads: blocks past the wave's share re-read its last block (cache hit) and
// are never used.
template <int NBW>
__device__ __forceinline__ void load_generic(GenRegs<NBW>& r, const int8_t* __restrict__ w,
                                             const uint16_t* __restrict__ sc, int row, int H, int nb, int bw0,
                                             int nbw, int g) {
    const int8_t* wp = w + (size_t)row * H + (size_t)bw0 * kBlock + g * 8;
    const uint16_t* sp = sc + (size_t)row * nb + bw0;
    const int last = nbw > 0 ? nbw - 1 : 0;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        const int b = i < last ? i : last;
        r.w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(wp + b * kBlock));
        r.sc[i] = sp[b];
    }
}

template <int MT, int NBW, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void q8b32_generic(GemmArgs a) {
    __shared__ f32x4 red[2][NW][MT][kWave];
    __shared__ f32x4 noise[EPI == EPI_SAMPLE ? 3 : 1][kWave];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int ks = blockIdx.y;
    const int kb0 = (int)((long long)a.nb * ks / a.ksplit);
    const int nbk = (int)((long long)a.nb * (ks + 1) / a.ksplit) - kb0;
    const int bw0 = kb0 + (int)((long long)nbk * wave / NW);
    const int nbw = kb0 + (int)((long long)nbk * (wave + 1) / NW) - bw0;

    f16x8 hid[NBW][MT];
    load_hidden<MT, NBW>(hid, a, bw0, nbw, n, g);
    Reducer<MT, NW, EPI> red_{red};
    red_.init();
    red_.noise = noise;
    red_.setup(a, wave, lane, blockIdx.x);                // items blockIdx.x, + grid, ...

    const int8_t* w = tile_up<EPI>(n) ? a.w1 : a.w0;
    const uint16_t* sc = tile_up<EPI>(n) ? a.s1 : a.s0;
    auto load = [&](GenRegs<NBW>& r, int item) {
        const int row = min(tile_row<EPI>(item, n), a.V - 1);     // tail rows re-read the last row; masked
        load_generic<NBW>(r, w, sc, row, a.H, a.nb, bw0, nbw, g);
    };
    auto process = [&](const GenRegs<NBW>& cur, int it, int buf) {
        red_.ahead(a, it + gridDim.x, wave, lane);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = zero;
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
            if (i < nbw) {
                const f16x8 b = i8x8_to_f16x8(cur.w[i]);
                const float s = h2f(cur.sc[i]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(hid[i][mt], b, zero, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[mt][r] = __builtin_fmaf(s, d[r], acc[mt][r]);
                }
            }
        }
        red_.run(a, acc, it, buf, wave, lane, ks);
    };

    const int step = gridDim.x;
    const int last = a.nitems - 1;
    GenRegs<NBW> ra, rb;
    int it = blockIdx.x;
    load(ra, it);
    while (true) {
        if (it >= a.nitems) break;
        load(rb, min(it + step, last));
        process(ra, it, 0);
        it += step;
        if (it >= a.nitems) break;
        load(ra, min(it + step, last));
        process(rb, it, 1);
        it += step;
    }
    if constexpr (EPI == EPI_HEAD || EPI == EPI_SAMPLE)
        if (a.ksplit == 1 && wave == 0) red_.finish(a, lane);
}

// ksplit > 1: sum the partial sums in split order, then apply the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void combine_kernel(GemmArgs a) {
    const int s = blockIdx.y;
    float bv = -INFINITY;
    int bi = INT_MAX;
    float run_m = -INFINITY, run_l = 0.0f;        // EPI_SAMPLE: online log-sum-exp of z
    uint32_t p0 = 0;
    int excl = -1;
    if constexpr (EPI == EPI_SAMPLE) {
        p0 = (uint32_t)a.state[SV_STATE_LEN];
        excl = s < a.S - 1 ? a.drafts[s] : -1;
    }
    for (int v = blockIdx.x * 256 + threadIdx.x; v < a.V; v += gridDim.x * 256) {
        const size_t o = (size_t)s * a.V + v;
        const size_t plane = (size_t)a.S * a.V;
        float t0 = a.kpart0[o];
        for (int k = 1; k < a.ksplit; ++k) t0 += a.kpart0[k * plane + o];
        if constexpr (EPI == EPI_HEAD) {
            if (a.logits) a.logits[o] = t0;
            if (t0 > bv) { bv = t0; bi = v; }
        } else if constexpr (EPI == EPI_SAMPLE) {
            // the sampling epilogue of the matmul, one element at a time
            if (a.logits) a.logits[o] = t0;
            const float z = t0 * a.inv_temp;
            const bool out = v == excl;
            if (out) a.zd[s] = z;
            const Philox4 rnd = philox4x32_10((uint32_t)v, p0, (uint32_t)(s >> 2), 0u, a.key0, a.key1);
            const float key = out ? -INFINITY : z + gumbel(uniform01(philox_word(rnd, s & 3)));
            if (key > bv) { bv = key; bi = v; }
            if (z > run_m) {
                run_l = run_l * __expf(run_m - z) + 1.0f;
                run_m = z;
            } else {
                run_l += __expf(z - run_m);
            }
        } else if constexpr (EPI == EPI_STORE) {
            if (a.residual) t0 += h2f(a.residual[o]);
            a.y[o] = f2h(t0);
        } else {
            float t1 = a.kpart1[o];
            for (int k = 1; k < a.ksplit; ++k) t1 += a.kpart1[k * plane + o];
            a.y[o] = f2h(t0 / (1.0f + expf(-t0)) * t1);
        }
    }
    if constexpr (EPI == EPI_HEAD || EPI == EPI_SAMPLE) {
        __shared__ float sv_[4], sm_[4], sl_[4];
        __shared__ int si_[4];
        argmax_group<64>(bv, bi);
        if constexpr (EPI == EPI_SAMPLE) lse_merge_group<64>(run_m, run_l);
        if ((threadIdx.x & 63) == 0) {
            sv_[threadIdx.x >> 6] = bv; si_[threadIdx.x >> 6] = bi;
            sm_[threadIdx.x >> 6] = run_m; sl_[threadIdx.x >> 6] = run_l;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 1; w < 4; ++w) {
                if (better(sv_[w], si_[w], bv, bi)) { bv = sv_[w]; bi = si_[w]; }
                lse_merge(run_m, run_l, sm_[w], sl_[w]);
            }
            a.part_val[(size_t)s * kGridMax + blockIdx.x] = bv;
            a.part_idx[(size_t)s * kGridMax + blockIdx.x] = bi;
            if constexpr (EPI == EPI_SAMPLE) {
                a.part_m[(size_t)s * kGridMax + blockIdx.x] = run_m;
                a.part_l[(size_t)s * kGridMax + blockIdx.x] = run_l;
            }
        }
    }
}

// Round tail, one workgroup of kTailThreads: reduce the per-workgroup argmax partials of the
// head launch in a fixed order into argmax[S] and, for a round (drafts_out != null), run the
// greedy accept and draft the next round.  The argmax is the critical path, so each wave's
// partial loads are issued first; the loads that do not depend on the argmax (state, drafts,
// the whole stream when it fits in LDS) follow at once, so the tail costs about one memory
// round trip; accept and drafter then work from LDS, behind barriers that order LDS only.
// A kernel boundary, not a device-scope fence in every matmul workgroup, orders the partials.
constexpr int kTailThreads = 1024;
constexpr int kTailIds = 32768;                      // stream ids the tail can hold in LDS (128 KB)
constexpr int kTailPart = 8;                         // partial loads in flight per lane and row
constexpr int kTailHead = 8192;                      // stream ids loaded before the length is known

__global__ __launch_bounds__(kTailThreads) void round_tail_kernel(const float* __restrict__ pv,
                                                                  const int* __restrict__ pi, int nparts, int S,
                                                                  int32_t* __restrict__ argmax,
                                                                  const int32_t* __restrict__ drafts_in,
                                                                  int32_t* __restrict__ tokens, int cap,
                                                                  int32_t* __restrict__ state, int nmax,
                                                                  int32_t* __restrict__ drafts_out) {
    __shared__ __attribute__((aligned(16))) int32_t tk[kTailIds + 8];    // + group reads past the end
    __shared__ int32_t am[SV_MAX_S];
    __shared__ int new_len;
    __shared__ int gated_s;
    __shared__ unsigned long long wbest[kTailThreads / kWave];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = S - 1;
    const bool round = drafts_out != nullptr;
    constexpr int kWaves = kTailThreads / kWave;
    // the stream length first (a scalar load): the stream beyond its first kTailHead ids is
    // loaded only up to it
    const int len_s = round ? state[SV_STATE_LEN] : 0;

    // the first kTailPart * 64 partials of this wave's first window row
    float v0[kTailPart];
    int i0[kTailPart];
#pragma unroll
    for (int u = 0; u < kTailPart; ++u) {
        const int p = u * kWave + lane;
        const bool ok = wave < S && p < nparts;
        v0[u] = ok ? pv[(size_t)wave * kGridMax + p] : -INFINITY;
        i0[u] = ok ? pi[(size_t)wave * kGridMax + p] : INT_MAX;
    }

    // then every other load that does not depend on the argmax: the stream's first
    // min(cap, kTailHead) ids (whatever its length), then the rest of the stream up to its length,
    // the state and the drafts; the stream goes to LDS once the partials are reduced
    int len0 = 0, d = -1;
    bool in_lds = false;
    IdPrefix<kTailHead / (4 * kTailThreads)> pre;
    IdPrefix<(kTailIds - kTailHead) / (4 * kTailThreads)> pre2;
    const int navail = round ? (cap < kTailIds ? cap : kTailIds) : 0;
    const int nhead = navail < kTailHead ? navail : kTailHead;
    const bool vec = round && (reinterpret_cast<uintptr_t>(tokens) & 15) == 0;
    if (vec) prefix_load(tokens, nhead, pre);
    StateCache sc{0, 0};
    if (round) {
        len0 = len_s;
        if (wave == 0) {
            sc = state_cache_load(state, lane);
            if (lane < K) d = drafts_in[lane];
        }
        in_lds = len0 >= 0 && len0 + K + 1 <= cap && len0 + K + 1 <= kTailIds;
    }
    for (int s = wave; s < S; s += kWaves) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int p0 = 0; p0 < nparts; p0 += kTailPart * kWave) {
            float v[kTailPart];
            int ix[kTailPart];
            if (s == wave && p0 == 0) {                                 // issued above
#pragma unroll
                for (int u = 0; u < kTailPart; ++u) { v[u] = v0[u]; ix[u] = i0[u]; }
            } else {
#pragma unroll
                for (int u = 0; u < kTailPart; ++u) {
                    const int p = p0 + u * kWave + lane;
                    v[u] = p < nparts ? pv[(size_t)s * kGridMax + p] : -INFINITY;
                    ix[u] = p < nparts ? pi[(size_t)s * kGridMax + p] : INT_MAX;
                }
            }
#pragma unroll
            for (int u = 0; u < kTailPart; ++u)
                if (better(v[u], ix[u], bv, bi)) { bv = v[u]; bi = ix[u]; }
        }
        argmax_group<64>(bv, bi);
        if (lane == 0) { argmax[s] = argmax_id(bi); am[s] = argmax_id(bi); }
    }
    if (!round) return;
    // the stream beyond its first kTailHead ids, up to its length (known by now)
    const int nrest = in_lds && len0 > kTailHead ? len0 : kTailHead;
    if (vec) prefix_load_from(tokens, kTailHead, nrest, pre2);
    if (in_lds) {
        if (vec) {
            prefix_store(tokens, nhead < len0 ? nhead : len0, pre, tk);
            prefix_store_from(tokens, kTailHead, nrest, pre2, tk);
            for (int i = ((len0 >> 2) << 2) + threadIdx.x; i < len0; i += kTailThreads)      // the ragged end
                if (i >= kTailHead) tk[i] = tokens[i];
        } else {
            stage_ids(tokens, len0, tk);
        }
    }
    if (!in_lds) {                                     // long or corrupt stream: the global-memory path
        __syncthreads();
        if (wave == 0) accept_wave(am, drafts_in, K, tokens, cap, state, lane);
        __syncthreads();                               // the drafter reads the stream and state just written
        propose_block(tokens, cap, state, nmax, K, drafts_out, tk, kTailIds - kHalo, wbest);
        return;
    }
    barrier_lds();
    if (wave == 0) {                                   // accept_wave, with the stream mirrored in LDS
        const unsigned long long hit = __ballot(lane < K && d >= 0 && d == am[lane < K ? lane : 0]);
        const int j = __builtin_ctzll(~hit);
        const int aj = am[j];
        if (aj < 0) {
            if (lane == 0) {
                state[SV_STATE_FLAGS] = state_word(sc, SV_STATE_FLAGS) | SV_FLAG_ARGMAX;
                new_len = len0;
                gated_s = state_word(sc, SV_STATE_GATED) != 0;
            }
        } else {
            if (lane < j) { tokens[len0 + lane] = d; tk[len0 + lane] = d; }
            if (lane == j) { tokens[len0 + j] = aj; tk[len0 + j] = aj; }
            const int gated = record_round_cached(sc, state, j, lane);
            if (lane == 0) {
                new_len = len0 + 1 + j;
                state[SV_STATE_LEN] = len0 + 1 + j;
                gated_s = gated != 0;
            }
        }
    }
    barrier_lds();                                     // the drafter reads only LDS (tk, new_len, gated_s)
    propose_lds(tk, new_len, nmax, K, drafts_out, state, wbest, gated_s != 0);
}

// ------------------------------------------------------------------------------------------
// shape tables (every instantiation compiles without register spills on gfx950)
// ------------------------------------------------------------------------------------------
typedef void (*KernelFn)(GemmArgs);
struct Shape { int mt, nbw, nw, epis, xr = 0; };
constexpr int kH = 1 << EPI_HEAD, kS = 1 << EPI_STORE, kG = 1 << EPI_GATEUP, kX = 1 << EPI_SAMPLE;

// fast kernel: every wave owns exactly nbw blocks (a multiple of 4); listed in order of
// preference within each MT; epis = the epilogues that compile for it without spills
// within the LDS limit
constexpr Shape kFast[] = {
    // order = preference where several shapes cover the hidden axis (measured: at H = 2048
    // 8 x 8 beats 4 x 16 for the argmax head, 80.6 against 82.9 us at S = 9, and loses for the
    // sampling head, 83.9 against 82.3 us; 8 x 10 beats 16 x 5 at H = 2560; 16 x 8 and 8 x 16
    // are even at H = 4096)
    {1, 8, 8, kH}, {1, 4, 16, kH | kS | kG | kX}, {1, 8, 8, kS | kG | kX}, {1, 8, 10, kH | kS | kG | kX},
    {1, 16, 5, kH | kS | kG | kX}, {1, 16, 8, kH | kS | kG | kX}, {1, 20, 8, kH | kS | kG | kX},
    {1, 8, 16, kH | kS}, {1, 16, 4, kH | kS | kG | kX}, {1, 8, 4, kH | kS | kG | kX},
    {1, 4, 4, kH | kS | kG | kX}, {1, 8, 2, kH | kS | kG | kX},
    {2, 8, 8, kH}, {2, 8, 5, kH}, {2, 8, 4, kH}, {2, 4, 4, kH},
    {4, 4, 4, kH},
    // S = 17: the one-tile kernel plus the 17th row's dot products (the shapes that compile
    // without spills; 20 blocks x 8 waves does not); 8 x 8 before 4 x 16 as for S <= 16
    {1, 8, 8, kH, 1}, {1, 4, 16, kH, 1}, {1, 16, 8, kH, 1}, {1, 16, 5, kH, 1}, {1, 8, 4, kH, 1}, {1, 4, 4, kH, 1},
    {1, 20, 8, kH, 1},              // window rows of 8 of the 20 blocks in LDS, one rolling register set
};
// generic kernel
constexpr Shape kGeneric[] = {
    {1, 4, 4, kH | kS | kG | kX}, {1, 8, 4, kH | kS | kG | kX}, {1, 16, 4, kH | kS | kG | kX},
    {1, 4, 8, kH | kS | kG | kX}, {1, 8, 8, kH | kS | kG | kX}, {1, 16, 8, kH | kS | kG | kX},
    {1, 4, 16, kH | kS | kX}, {1, 8, 16, kH | kS},
    {2, 4, 4, kH}, {2, 8, 4, kH}, {2, 4, 8, kH}, {2, 8, 8, kH},
    {4, 2, 4, kH}, {4, 4, 4, kH}, {4, 2, 8, kH},
};

template <int EPI>
KernelFn pick_fast(const GemmCfg& c) {
    if constexpr (EPI == EPI_HEAD) {
        if (c.xr) {
#define SV_XR(NBW, NW, XR) \
    if (c.mt == 1 && c.xr == XR && c.nbw == NBW && c.nw == NW) return q8b32_fast<1, NBW, NW, EPI, XR>;
            SV_XR(4, 16, 1) SV_XR(8, 8, 1) SV_XR(16, 8, 1) SV_XR(16, 5, 1) SV_XR(8, 4, 1) SV_XR(4, 4, 1)
            // one rolling register set: window rows of 8 of the 20 blocks in LDS (12 with two
            // sets); measured 198 against 239 us at 248320 x 5120, S = 17
            if (c.mt == 1 && c.xr == 1 && c.nbw == 20 && c.nw == 8) return q8b32_fast<1, 20, 8, EPI, 1, 8, 1>;
#undef SV_XR
            return nullptr;
        }
    }
    if (c.xr) return nullptr;
#define SV_SHAPE(MT, NBW, NW) \
    if (c.mt == MT && c.nbw == NBW && c.nw == NW) return q8b32_fast<MT, NBW, NW, EPI>;
    // the argmax head at 8 x 10 (H = 2560) with one rolling register set: 63.2 against 64.4 us
    // at 151936 x 2560; at the other shapes two sets measured even or faster
    if constexpr (EPI == EPI_HEAD)
        if (c.mt == 1 && c.nbw == 8 && c.nw == 10) return q8b32_fast<1, 8, 10, EPI, 0, 0, 1>;
    SV_SHAPE(1, 8, 8) SV_SHAPE(1, 8, 10) SV_SHAPE(1, 16, 8) SV_SHAPE(1, 16, 5) SV_SHAPE(1, 16, 4)
    SV_SHAPE(1, 8, 4) SV_SHAPE(1, 4, 4) SV_SHAPE(1, 8, 2) SV_SHAPE(1, 4, 16) SV_SHAPE(1, 20, 8)
    if constexpr (EPI == EPI_HEAD || EPI == EPI_STORE) { SV_SHAPE(1, 8, 16) }
    if constexpr (EPI == EPI_HEAD) {
        SV_SHAPE(2, 8, 8) SV_SHAPE(2, 8, 5) SV_SHAPE(2, 8, 4) SV_SHAPE(2, 4, 4) SV_SHAPE(4, 4, 4)
    }
#undef SV_SHAPE
    return nullptr;
}

template <int EPI>
KernelFn pick_generic(const GemmCfg& c) {
#define SV_SHAPE(MT, NBW, NW) \
    if (c.mt == MT && c.nbw == NBW && c.nw == NW) return q8b32_generic<MT, NBW, NW, EPI>;
    SV_SHAPE(1, 4, 4) SV_SHAPE(1, 8, 4) SV_SHAPE(1, 16, 4) SV_SHAPE(1, 4, 8) SV_SHAPE(1, 8, 8) SV_SHAPE(1, 16, 8)
    if constexpr (EPI != EPI_GATEUP) { SV_SHAPE(1, 4, 16) }
    if constexpr (EPI == EPI_HEAD || EPI == EPI_STORE) { SV_SHAPE(1, 8, 16) }
    if constexpr (EPI == EPI_HEAD) {
        SV_SHAPE(2, 4, 4) SV_SHAPE(2, 8, 4) SV_SHAPE(2, 4, 8) SV_SHAPE(2, 8, 8)
        SV_SHAPE(4, 2, 4) SV_SHAPE(4, 4, 4) SV_SHAPE(4, 2, 8)
    }
#undef SV_SHAPE
    return nullptr;
}

// Fast shape: the hidden axis splits into ks equal parts, each into nw waves of exactly
// nbw blocks.
bool try_fast(int nb, int mt, int epi, GemmCfg& c, int xr = 0) {
    for (int ks = 1; ks <= 8; ++ks) {
        if (nb % ks) continue;
        const int nbk = nb / ks;
        for (const Shape& sh : kFast) {
            if (sh.mt != mt || sh.xr != xr || !(sh.epis & (1 << epi))) continue;
            if (g_nw_override && sh.nw != g_nw_override) continue;
            if (sh.nbw * sh.nw == nbk) {
                c.mt = mt; c.nbw = sh.nbw; c.nw = sh.nw; c.ksplit = ks; c.fast = 1; c.xr = xr;
                return true;
            }
        }
    }
    return false;
}

bool try_generic(int nb, int mt, int epi, int nw_fixed, GemmCfg& c) {
    const int pref[3] = {8, 16, 4};
    for (int ks = 1; ks <= nb; ++ks) {
        const int nbk = (nb + ks - 1) / ks;
        for (int t = 0; t < 3; ++t) {
            const int nw = nw_fixed ? nw_fixed : (nb < 32 ? 4 : pref[t]);
            const int need = (nbk + nw - 1) / nw;
            int best = 0;
            for (const Shape& sh : kGeneric)
                if (sh.mt == mt && (sh.epis & (1 << epi)) && sh.nw == nw && sh.nbw >= need &&
                    (best == 0 || sh.nbw < best))
                    best = sh.nbw;
            if (best) {
                c.mt = mt; c.nbw = best; c.nw = nw; c.ksplit = ks; c.fast = 0;
                return true;
            }
            if (nw_fixed || nb < 32) break;
        }
    }
    return false;
}

KernelFn kernel_for(int epi, const GemmCfg& c) {
    if (c.fast) {
        if (epi == EPI_HEAD) return pick_fast<EPI_HEAD>(c);
        if (epi == EPI_SAMPLE) return pick_fast<EPI_SAMPLE>(c);
        if (epi == EPI_STORE) return pick_fast<EPI_STORE>(c);
        return pick_fast<EPI_GATEUP>(c);
    }
    if (epi == EPI_HEAD) return pick_generic<EPI_HEAD>(c);
    if (epi == EPI_SAMPLE) return pick_generic<EPI_SAMPLE>(c);
    if (epi == EPI_STORE) return pick_generic<EPI_STORE>(c);
    return pick_generic<EPI_GATEUP>(c);
}

// Workgroups of this kernel resident on the whole device at once.  Without a device to ask
// (no GPU, or a failed query) the answer is one 16-wave group or two smaller groups per
// compute unit of a 256-CU part; it only sizes the grid, never a buffer.
int resident_groups(int epi, const GemmCfg& c) {
    struct Entry { KernelFn fn; int dev; int groups; };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    KernelFn fn = kernel_for(epi, c);
    int dev = -1;
    const int fallback = c.nw >= 16 ? 256 : 512;
    if (!fn || hipGetDevice(&dev) != hipSuccess) return fallback;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].groups;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), c.nw * 64, 0) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1) {
        (void)hipGetLastError();
        return fallback;
    }
    const int groups = per_cu * cus;
    if (used < 64) cache[used++] = Entry{fn, dev, groups};
    return groups;
}

}  // namespace

int tuning_waves() { return g_nw_override; }
int tuning_groups() { return g_grid_override; }

void set_tuning(int waves_per_group, int max_groups, int no_extra_row) {
    g_nw_override = waves_per_group;
    g_grid_override = max_groups;
    g_no_xr = no_extra_row;
}

GemmCfg gemm_config(int rows, int H, int S, int epi) {
    GemmCfg c{};
    const int mt = S <= 16 ? 1 : (S <= 32 ? 2 : 4);
    const int nb = H / kBlock;
    // The fast loads stream at about twice the generic ones, so the fast kernel wins unless it
    // needs more than one extra workgroup split of the hidden axis (each split adds partial
    // sums and a combine pass); an unsplit generic launch beats any split one.
    GemmCfg f{}, gen{};
    // 17 .. 20 window rows: the fast kernel with rows 16+ in LDS, unsplit, when a shape fits
    bool have_fast = false;
    if (epi == EPI_HEAD && S == 17 && !g_no_xr) {
        have_fast = try_fast(nb, 1, epi, f, 1);
        if (have_fast && f.ksplit > 1) have_fast = false;
    }
    if (!have_fast) have_fast = try_fast(nb, mt, epi, f);
    if (!(g_nw_override && try_generic(nb, mt, epi, g_nw_override, gen)))
        try_generic(nb, mt, epi, 0, gen);     // always succeeds: (mt, smallest nbw, 4 waves) exists
    const bool take_fast = have_fast && (f.ksplit == 1 || (gen.ksplit > 1 && f.ksplit <= gen.ksplit + 1));
    c = take_fast ? f : gen;
    // Persistent grid: as many workgroups as the chip holds at once (the register and LDS
    // footprint of the chosen kernel decide how many fit on a compute unit), so no
    // workgroup waits for another to retire and every one keeps its loads in flight.
    const int items = epi == EPI_GATEUP ? (rows + 7) / 8 : (rows + kTileRows - 1) / kTileRows;
    int cap = g_grid_override ? g_grid_override : resident_groups(epi, c) / c.ksplit;
    if (cap < 1) cap = 1;
    if (cap > kGridMax) cap = kGridMax;
    // Balanced: every workgroup gets the same number of items (+-1 only when the items do not
    // divide), so no single workgroup runs an extra item after the others have finished.
    const int per = (items + cap - 1) / cap;
    c.grid = items > 0 ? (items + per - 1) / per : 1;
    // One contiguous range of items per die for the one-tile fast argmax head over rows of at
    // most 2 KB, the grid rounded up to a multiple of kXcds within the resident cap.  Measured,
    // head alone, alternating builds on one device each: 248320 x 2048 at S = 9 82.2-83.0
    // against 85.3-86.3 us (80.2-80.6 against 80.9-81.8 us on another device) and at S = 17
    // 81.7-83.1 against 84.3-85.0 us; the fused round at that shape 86.1-86.5 against
    // 87.2-87.4 us.  At H = 2560 and 5120 it measured 0.5% slower and at 4096 even, the int4
    // head gained nothing, and the sampling head (4 x 16 shape, one workgroup per compute unit)
    // ran 4% slower with it (c3samp rounds), so those keep the interleaved order.  The kernels
    // read xcd for EPI_HEAD only: the sampling kernel built with the runtime choice ran 3% slower
    // even in the interleaved order.
    c.xcd = 0;
    if (c.fast && c.mt == 1 && c.ksplit == 1 && epi == EPI_HEAD && H <= 2048) {
        const int g8 = (c.grid + kXcds - 1) / kXcds * kXcds;
        if (c.grid >= kXcds && g8 <= cap && items >= kXcds * g8) {
            c.grid = g8;
            c.xcd = 1;
        }
    }
    return c;
}

int combine_groups(int V) {
    const int g = (V + 255) / 256;
    return g < 256 ? g : 256;
}

// More than 32 window rows: the four-tile shapes cover the hidden axis only by splitting it
// across workgroups (their window rows and cross-wave sums outgrow the registers and LDS of
// one workgroup), and a split head writes and re-reads 4 x ks x S x V bytes of fp32 partial
// sums.  Two passes of an unsplit two-tile shape read the weights twice instead and keep every
// dot product whole (measured at 248320 x 2048: 187 us for both passes against 236-283 us
// split at S = 33 .. 64).
GemmCfg head_config(int V, int H, int S, int& passes) {
    passes = 1;
    if (S > 32) {
        const GemmCfg c = gemm_config(V, H, 32, EPI_HEAD);
        if (c.fast && c.ksplit == 1) {
            passes = 2;
            return c;
        }
    }
    return gemm_config(V, H, S, EPI_HEAD);
}

size_t head_workspace_bytes(int V, int H, int S) {
    int passes = 1;
    const GemmCfg c = head_config(V, H, S, passes);
    size_t b = head_partials_bytes(S);
    if (c.ksplit > 1) b += (size_t)4 * c.ksplit * S * V;
    return b;
}

size_t sample_workspace_bytes(int V, int H, int S) {
    const GemmCfg c = gemm_config(V, H, S, EPI_SAMPLE);
    size_t b = 2 * head_partials_bytes(S) + 256;
    if (c.ksplit > 1) b += (size_t)4 * c.ksplit * S * V;
    return b;
}

size_t stack_workspace_bytes(int N, int K, int S, bool gateup) {
    const GemmCfg c = gemm_config(N, K, S, gateup ? EPI_GATEUP : EPI_STORE);
    if (c.ksplit == 1) return 0;
    return (size_t)4 * c.ksplit * S * N * (gateup ? 2 : 1);
}

hipError_t launch_q8b32(int epi, const GemmCfg& cfg, const GemmArgs& a, hipStream_t stream, bool combine,
                        hipEvent_t start, hipEvent_t stop) {
    KernelFn fn = kernel_for(epi, cfg);
    if (!fn) return hipErrorInvalidConfiguration;
    const bool split = cfg.ksplit > 1 && combine;
    GemmArgs ka = a;
    ka.xcd = cfg.xcd;
    launch_timed(fn, dim3(cfg.grid, cfg.ksplit), dim3(cfg.nw * 64), stream, start, split ? nullptr : stop, ka);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    const int cg = combine_groups(a.V);
    const dim3 grid(cg, a.S), block(256);
    if (epi == EPI_HEAD)
        launch_timed(combine_kernel<EPI_HEAD>, grid, block, stream, nullptr, stop, a);
    else if (epi == EPI_SAMPLE)
        launch_timed(combine_kernel<EPI_SAMPLE>, grid, block, stream, nullptr, stop, a);
    else if (epi == EPI_STORE)
        launch_timed(combine_kernel<EPI_STORE>, grid, block, stream, nullptr, stop, a);
    else
        launch_timed(combine_kernel<EPI_GATEUP>, grid, block, stream, nullptr, stop, a);
    return hipGetLastError();
}

hipError_t launch_round_tail(const float* pv, const int* pi, int nparts, int S, int32_t* argmax,
                             const int32_t* drafts_in, int32_t* tokens, int cap, int32_t* state, int nmax,
                             int32_t* drafts_out, hipStream_t stream) {
    hipLaunchKernelGGL(round_tail_kernel, dim3(1), dim3(kTailThreads), 0, stream, pv, pi, nparts, S, argmax,
                       drafts_in, tokens, cap, state, nmax, drafts_out);
    return hipGetLastError();
}

}  // namespace sv
