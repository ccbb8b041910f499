// Int4 per-block-32 head matmul for gfx950 with the fused argmax (stage 1).
//
// Pages: "Riding Apple's pipelined GPU engine", section "Quantization on the GPU delegate"
// (int4 linear per-block-32 is the int4 class that ships; per-block linear dequant beats a
// LUT at the same bytes) and section "Numerics gating" (QAT q4_0 weights follow the
// per-block-32 absmax grid).  Half the weight bytes of the int8 head for the same logits
// class:
//   L[s, v] = sum_b f32(scale[v, b]) * sum_{k in block b} f32(code[v, k]) * f32(x[s, k])
// Storage per 32-block: 16 bytes, byte i = element i (low nibble) | element i+16 (high
// nibble) << 4, offset binary (code = nibble - 8, codes -7 .. 7).
//
// Mapping (same MFMA as the int8 head, v_mfma_f32_16x16x32_f16, one block per instruction).
// The MFMA sums over its 32 k slots, so any fixed assignment of a block's elements to slots
// works if the A operand (window rows) and the B operand (codes) use the same one.  Lane l
// (row n = l % 16, group g = l / 16) reads ONE dword of its row's block, bytes 4g .. 4g+3:
// their low nibbles are elements 4g .. 4g+3, their high nibbles elements 16+4g .. 16+4g+3,
// placed in the slot order of nib8_to_f16x8; the held window rows are loaded in that same
// order.  A nibble placed under the fp16 exponent of 1024 is 1024 + nibble exactly (1024 + 16 x
// nibble for a high nibble); an fp16 subtract (or scale and subtract) leaves the code.  Each wave loads 8 rows x 128 contiguous bytes
// per instruction (8 int4 blocks of each row) and exchanges them into the MFMA layout through
// its own two 2 KB LDS slots, 16-byte chunks XOR-swizzled by row (one chunk is one block).
// The block scale is applied to the MFMA result one block later, so no instruction waits on
// a just-issued MFMA.  A workgroup owns 16 vocab rows at a time; its NW waves split the
// hidden axis (NBW blocks each) and reduce through LDS in a fixed order; wave w then keeps the
// running (value, lowest index) of window rows w, w + NW, ...  The next two items' loads are
// in flight during the current item's math.
#include "sv_device.h"
#include "sv_internal.h"

#include <climits>
#include <cmath>
#include <mutex>

namespace sv {

namespace {

__device__ __forceinline__ void lds_barrier_q4() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One dword of a block (bytes 4g .. 4g+3) -> its 8 codes in slot order
//   slots 0..7 = elements 4g, 4g+2, 4g+1, 4g+3, 16+4g, 16+4g+2, 16+4g+1, 16+4g+3.
// Each half-word of the dword holds two bytes; masking one nibble of each half and OR-ing the
// fp16 exponent of 1024 gives 1024 + nibble (a low nibble) or 1024 + 16 * nibble (a high
// nibble, mantissa bits 4..7), both exact; subtracting 1032, or scaling by 1/16 and
// subtracting 72, leaves the code exactly.  Nine instructions for eight codes.
// (w & mask) | exponent as one v_bfi_b32 (the compiler otherwise emits an AND and an OR);
// the mask in a scalar register, the exponent pattern in a vector one (one scalar operand
// per instruction on this architecture).
__device__ __forceinline__ uint32_t nib_under_exp(uint32_t w, uint32_t mask, uint32_t expo) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(w), "v"(expo));
    return r;
}

__device__ __forceinline__ f16x8 nib8_to_f16x8(uint32_t w) {
    const f16x2 bias_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const f16x2 bias_hi = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    const uint32_t expo = 0x64006400u;
    const f16x2 e02 = __builtin_bit_cast(f16x2, nib_under_exp(w, 0x000F000Fu, expo)) - bias_lo;
    const f16x2 e13 = __builtin_bit_cast(f16x2, nib_under_exp(w8, 0x000F000Fu, expo)) - bias_lo;
    const f16x2 h02 = __builtin_bit_cast(f16x2, nib_under_exp(w, 0x00F000F0u, expo)) * sixteenth + bias_hi;
    const f16x2 h13 = __builtin_bit_cast(f16x2, nib_under_exp(w8, 0x00F000F0u, expo)) * sixteenth + bias_hi;
    f16x8 r;
    r[0] = e02[0]; r[1] = e02[1]; r[2] = e13[0]; r[3] = e13[1];
    r[4] = h02[0]; r[5] = h02[1]; r[6] = h13[0]; r[7] = h13[1];
    return r;
}

template <int NBW>
struct Q4Regs {
    static constexpr int NSEG = NBW / 8;           // 128-byte segments (8 int4 blocks) per row per wave
    u32x4 w[NSEG][2];                              // [segment][row half]
    uint32_t sc[NBW / 2];                          // fp16 scales of the lane's row, in pairs
};

// ROLL = 0: three fixed register sets (two items' loads in flight while one is converted);
// ROLL = k > 0: k sets refilled segment by segment as the LDS exchange frees them.
template <int NBW, int NW, int ROLL = 0>
__global__ __launch_bounds__(NW * 64) void q4b32_head(Q4Args a) {
    constexpr int NSEG = NBW / 8;
    static_assert(NBW % 8 == 0, "whole 128-byte segments");
    __shared__ f32x4 red[2][NW][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t xch[NW][2][2048];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int bw0 = NBW * wave;                    // first block of this wave
    const int row_bytes = a.H / 2;

    // window rows in slot order: elements 4g, 4g+2, 4g+1, 4g+3, then the same four + 16
    f16x8 hid[NBW];
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
        f16x8 h = {};
        if (n < a.S) {
            const uint16_t* xb = a.x + (size_t)n * a.H + (size_t)(bw0 + i) * kBlock + 4 * g;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(xb);        // elements 4g .. 4g+3
            const u32x2 hi = *reinterpret_cast<const u32x2*>(xb + 16);   // elements 16+4g .. 16+4g+3
            const u32x4 q = {__builtin_amdgcn_perm(lo.y, lo.x, 0x05040100u), __builtin_amdgcn_perm(lo.y, lo.x, 0x07060302u),
                             __builtin_amdgcn_perm(hi.y, hi.x, 0x05040100u), __builtin_amdgcn_perm(hi.y, hi.x, 0x07060302u)};
            h = __builtin_bit_cast(f16x8, q);
        }
        hid[i] = h;
    }
    // epilogue spread over the waves: wave w finishes window rows w, w + NW, ... (lanes 0-15
    // hold the 16 vocab rows of the item), so no wave trails the others at each item's barrier
    constexpr int RPW = (16 + NW - 1) / NW;
    float best_v[RPW];
    int best_i[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) { best_v[j] = -INFINITY; best_i[j] = INT_MAX; }

    const int lrow = lane >> 3, lchunk = lane & 7;
    auto load_seg = [&](Q4Regs<NBW>& r, int item, int t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = min(item * kTileRows + 8 * h + lrow, a.V - 1);       // tail rows: masked later
            const uint8_t* p = a.w + (size_t)row * row_bytes + (size_t)bw0 * 16 + 16 * lchunk;
            r.w[t][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 128 * t));
        }
    };
    auto load_sc = [&](Q4Regs<NBW>& r, int item) {
        const int srow = min(item * kTileRows + n, a.V - 1);
        const uint16_t* sp = a.s + (size_t)srow * a.nb + bw0;
#pragma unroll
        for (int v = 0; v < NBW / 8; ++v) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(sp + 8 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.sc[4 * v + e] = q[e];
        }
    };
    auto load = [&](Q4Regs<NBW>& r, int item) {
#pragma unroll
        for (int t = 0; t < NSEG; ++t) load_seg(r, item, t);
        load_sc(r, item);
    };

    // nxt: with ROLL, the item whose loads replace cur's registers as they free up
    auto process = [&](Q4Regs<NBW>& cur, int it, int buf, int nxt) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc = zero;
        f32x4 dprev = zero;
        float scprev = 0.f;
#pragma unroll
        for (int t = 0; t < NSEG; ++t) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 8 * h + lrow;
                *reinterpret_cast<u32x4*>(&xch[wave][t & 1][row * 128 + 16 * (lchunk ^ (row & 7))]) = cur.w[t][h];
            }
            if constexpr (ROLL) load_seg(cur, nxt, t);
#pragma unroll
            for (int bb = 0; bb < 8; ++bb) {                     // 8 int4 blocks per segment
                const int i = 8 * t + bb;
                const int off = n * 128 + 16 * (bb ^ (n & 7)) + 4 * g;
                const uint32_t q4 = *reinterpret_cast<const uint32_t*>(&xch[wave][t & 1][off]);
                const f16x8 b = nib8_to_f16x8(q4);
                const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(hid[i], b, zero, 0, 0, 0);
                // the previous block's result is ready by now: scale and accumulate it
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(scprev, dprev[r], acc[r]);
                dprev = d;
                scprev = h2f((uint16_t)(cur.sc[i >> 1] >> (16 * (i & 1))));
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(scprev, dprev[r], acc[r]);
        if constexpr (ROLL) load_sc(cur, nxt);
        red[buf][wave][lane] = acc;
        lds_barrier_q4();
        const int v = it * kTileRows + n;
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int s = wave + j * NW;
            if (s >= a.S || s >= 16) break;                      // wave-uniform
            // D[s][n] of every wave sits in lane n + 16 * (s / 4), component s % 4
            const float* col = reinterpret_cast<const float*>(&red[buf][0][n + 16 * (s >> 2)]) + (s & 3);
            float val = col[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) val += col[w * kWave * 4];
            if (lane < 16 && v < a.V) {
                if (a.logits) a.logits[(size_t)s * a.V + v] = val;
                if (val > best_v[j]) { best_v[j] = val; best_i[j] = v; }
            }
        }
    };

    const int step = gridDim.x;
    const int last = a.nitems - 1;
    int it = blockIdx.x, k = 0;
    if constexpr (ROLL) {
        // ROLL register sets refilled segment by segment: set j holds items j, j + ROLL, ...,
        // so ROLL items' loads are in flight
        Q4Regs<NBW> rs[ROLL];
#pragma unroll
        for (int j = 0; j < ROLL; ++j) load(rs[j], min(it + j * step, last));
        while (it < a.nitems) {
#pragma unroll
            for (int j = 0; j < ROLL; ++j) {
                if (it < a.nitems) process(rs[j], it, k++ & 1, min(it + ROLL * step, last));
                it += step;
            }
        }
    } else {
        // three register sets: two items' loads stay in flight while one is processed
        Q4Regs<NBW> ra, rb, rc;
        load(ra, it);
        load(rb, min(it + step, last));
        while (true) {
            if (it >= a.nitems) break;
            load(rc, min(it + 2 * step, last));
            process(ra, it, k++ & 1, 0);
            it += step;
            if (it >= a.nitems) break;
            load(ra, min(it + 2 * step, last));
            process(rb, it, k++ & 1, 0);
            it += step;
            if (it >= a.nitems) break;
            load(rb, min(it + 2 * step, last));
            process(rc, it, k++ & 1, 0);
            it += step;
        }
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        const int s = wave + j * NW;
        if (s >= a.S || s >= 16) break;
        float bv = best_v[j];
        int bi = best_i[j];
        argmax_group<16>(bv, bi);
        if (lane == 0) {
            a.part_val[(size_t)s * kGridMax + blockIdx.x] = bv;
            a.part_idx[(size_t)s * kGridMax + blockIdx.x] = bi;
        }
    }
}

typedef void (*Q4Fn)(Q4Args);

// (blocks per wave, waves) -> kernel
Q4Fn pick_q4(int nbw, int nw) {
// 8-block waves in workgroups of up to 8 waves keep one rolling register set: 80 registers,
// so three 8-wave workgroups fit on a compute unit instead of two (measured at 248320 x 2048:
// 55.0 against 57.8 us with three fixed sets); wider workgroups keep the three sets.  More
// rolling sets keep more items in flight but fewer waves: 2 sets measured even, 3 and 4 sets
// 1.5% and 4.5% slower.
constexpr int kQ4Sets = 1;
#define SV_Q4(NBW, NW) \
    if (nbw == NBW && nw == NW) return q4b32_head<NBW, NW, (NBW == 8 && NW <= 8) ? kQ4Sets : 0>;
    SV_Q4(8, 1) SV_Q4(8, 2) SV_Q4(8, 4) SV_Q4(8, 5) SV_Q4(8, 6) SV_Q4(8, 8) SV_Q4(8, 10) SV_Q4(8, 12)
    SV_Q4(8, 14) SV_Q4(8, 16)
    SV_Q4(16, 4) SV_Q4(16, 5) SV_Q4(16, 6) SV_Q4(16, 8) SV_Q4(16, 10) SV_Q4(16, 12)   // 14, 16 spill
#undef SV_Q4
    return nullptr;
}

int q4_resident(Q4Fn fn, int nw) {
    struct Entry { Q4Fn fn; int dev; int groups; };
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

// Shape: every wave owns 8 (preferred) or 16 whole blocks; false when no instantiated
// (blocks per wave, waves) pair covers H exactly.
bool q4_config(int V, int H, Q4Cfg& c) {
    if (H % 256) return false;
    const int nb = H / kBlock;
    for (int nbw : {8, 16}) {
        const int nw = nb / nbw;
        if (nb % nbw || nw < 1 || nw > 16) continue;
        if (tuning_waves() && nw != tuning_waves()) continue;     // the calling thread's override
        Q4Fn fn = pick_q4(nbw, nw);
        if (!fn) continue;
        c.nbw = nbw;
        c.nw = nw;
        const int items = (V + kTileRows - 1) / kTileRows;
        int cap = q4_resident(fn, nw);
        if (tuning_groups() > 0) cap = tuning_groups();
        if (cap > kGridMax) cap = kGridMax;
        const int per = (items + cap - 1) / cap;
        c.grid = (items + per - 1) / per;
        c.items = items;
        return true;
    }
    return false;
}

hipError_t launch_q4(const Q4Cfg& c, const Q4Args& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    Q4Fn fn = pick_q4(c.nbw, c.nw);
    if (!fn) return hipErrorInvalidConfiguration;
    launch_timed(fn, dim3(c.grid), dim3(c.nw * 64), stream, start, stop, a);
    return hipGetLastError();
}

}  // namespace sv
