// fp32 attention forward for gfx950: same online-softmax recurrence and
// register layouts as the 16-bit kernel (mha_fwd16.hpp), on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32), so no input is ever rounded below fp32.
//
// One 4-wave workgroup per (query tile, batch, group of hp heads sharing a
// K/V head); each wave owns 32 query rows of one head, so a query tile is
// 128 / hp rows; key tiles of 32 keys.
//  * S^T = K Q^T: for k-step s (0 .. D/2-1) lane (c, g) supplies
//    Q[row c][dsel(s, g)] and K[key c][dsel(s, g)], dsel(s, g) =
//    s%H + 2H(s/H) + Hg with H = min(32, D/2) (any split of d between the
//    two lane halves works; this one keeps each half's Q values contiguous
//    in runs of H).
//  * The accumulator element 4i+j of lane (c, g) is key 8i + 4g + j of
//    query c, which is directly the B operand (one key per k-step) of
//    O^T = V^T P^T; V is read from LDS one fp32 per lane per k-step.
//  * K and V go global -> registers -> LDS (double buffered); K rows are
//    padded to an odd stride and V rows to D + 8 so the LDS reads of one
//    wave hit distinct banks.
//  * Key split (SPLIT, calls with few work items, head dim <= 64): a
//    workgroup owns 32 query rows of one head, and its four waves take
//    every fourth key tile each, each staging its own tiles in its own LDS
//    block (no workgroup barrier in the key loop). At the end the four
//    partial states (m, l, O) are merged exactly, as the online softmax
//    merges tiles: O = sum_w 2^(m_w - M) O_w, l likewise, M = max_w m_w.
//    This shortens the serial MFMA chain of each wave fourfold, which is
//    what bounds a call with fewer workgroups than compute units.
#pragma once

#include "mha_common.hpp"

namespace fa355 {

constexpr int kThreads32 = 256;  // 4 waves of 64 lanes
constexpr int kWaves32 = kThreads32 / 64;  // 32 query rows each

template <int D>
struct Tile32 {
    static constexpr int BN = 32;       // keys per tile
    static constexpr int ND = D / 32;   // 32-dim sub-tiles of O^T
    static constexpr int H = D < 64 ? D / 2 : 32;  // dsel run length
    static constexpr int K_LD = D + 1;  // LDS row strides (floats)
    static constexpr int V_LD = D + 8;
    static constexpr int K_ELEMS = BN * K_LD;
    static constexpr int STAGE = K_ELEMS + BN * V_LD;
    // At D = 256 the Q fragments and O^T take 256 registers: one wave per SIMD.
    static constexpr int WPE = D == 256 ? 1 : 2;
    static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dim");
};

// Head dims whose key-split instance is built (per-wave staging of a whole
// tile takes D / 2 registers per lane, and four single-buffered tiles fit
// in LDS).
constexpr bool split_dim32(int D) { return D <= 64; }

template <int D, int MASK, bool SPLIT>
__global__ __launch_bounds__(kThreads32) __attribute__((amdgpu_waves_per_eu(Tile32<D>::WPE, Tile32<D>::WPE)))
void mha_fwd32(Params p)
{
    using TL = Tile32<D>;
    constexpr int BN = TL::BN;
    constexpr int ND = TL::ND;
    static_assert(!SPLIT || split_dim32(D), "key split is built for head dims up to 64");

    // Normal: two stages shared by the workgroup. Key split: one stage per wave.
    __shared__ __attribute__((aligned(16))) float lds[(SPLIT ? kWaves32 : 2) * TL::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c32 = lane & 31;
    const int g = lane >> 5;

    const TileCoord tc = block_coord(blockIdx.x, p.n_qtiles, p.B, p.H, p.Hkv, p.hp, 0);
    const int b = tc.b, kvh = tc.h / p.rep;
    const int h = SPLIT ? tc.h : tc.h + wave / p.wph;  // this wave's query head
    const int rows = SPLIT ? 32 : 32 * p.wph;         // query rows per head in this workgroup
    const int S = p.S, W = p.window;
    const int q0 = tc.qt * rows;
    const int wrow0 = SPLIT ? q0 : q0 + (wave % p.wph) * 32;
    const int row = wrow0 + c32;  // this lane's query row

    const float *__restrict__ Q = static_cast<const float *>(p.q);
    const float *__restrict__ K = static_cast<const float *>(p.k);
    const float *__restrict__ V = static_cast<const float *>(p.v);
    float *__restrict__ O = static_cast<float *>(p.out);

    const int64_t q_row_stride = (int64_t)p.H * D;
    const int64_t kv_row_stride = (int64_t)p.Hkv * D;
    const float *Kbh = K + (int64_t)b * S * kv_row_stride + (int64_t)kvh * D;
    const float *Vbh = V + (int64_t)b * S * kv_row_stride + (int64_t)kvh * D;

    // Q fragments: qf[s/4][s%4] = Q[row][dsel(s, g)]. Rows past the end of
    // the sequence read the last row (their results are never stored).
    constexpr int NQ = D / 8;
    u32x4 qf[NQ];
    {
        const float *qrow = Q + ((int64_t)b * S + min(row, S - 1)) * q_row_stride + (int64_t)h * D;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            const int d = (4 * s) % TL::H + 2 * TL::H * ((4 * s) / TL::H) + TL::H * g;
            qf[s] = ldg16(qrow + d) ^ p.q_sign;
        }
    }

    int kt_begin, kt_end;
    key_tile_range<MASK, BN>(q0, rows, S, W, kt_begin, kt_end);

    // Staging: every thread moves D/32 rows x 16 bytes of K and of V (key
    // split: each wave moves its own tiles, D/8 rows per lane).
    constexpr int STAGERS = SPLIT ? 64 : kThreads32;
    const int sid = SPLIT ? lane : tid;
    float *const stage0 = lds + (SPLIT ? wave * TL::STAGE : 0);
    constexpr int CPR = D / 4;
    constexpr int STEP = STAGERS / CPR;
    constexpr int R = BN / STEP;
    u32x4 stg[2 * R];
    auto load_tile = [&](int kt) {
        const int k0 = kt * BN;
        const int c = sid % CPR, kr = sid / CPR;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int key = min(k0 + kr + r * STEP, S - 1);  // rows past S are masked
            stg[r] = ldg16(Kbh + (int64_t)key * kv_row_stride + 4 * c);
            stg[R + r] = ldg16(Vbh + (int64_t)key * kv_row_stride + 4 * c);
        }
    };
    auto store_tile = [&](int buf) {
        float *Ks = stage0 + buf * TL::STAGE;
        float *Vs = Ks + TL::K_ELEMS;
        const int c = sid % CPR, kr = sid / CPR;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int key = kr + r * STEP;
            float *kd = Ks + key * TL::K_LD + 4 * c;
#pragma unroll
            for (int e = 0; e < 4; ++e) kd[e] = __uint_as_float(stg[r][e]);
            *reinterpret_cast<u32x4 *>(Vs + key * TL::V_LD + 4 * c) = stg[R + r];
        }
    };

    f32x16 oacc[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) oacc[t] = f32x16{};
    float m_run = -INFINITY;  // running max, in scaled log2 units
    float l_run = 0.0f;       // this lane's share of the running sum
    const float sl2e = p.scale_log2;

    // Key tiles of this wave: all of the workgroup's, or (key split) every
    // fourth one from kt_begin + wave.
    const int kt_first = SPLIT ? kt_begin + wave : kt_begin;
    constexpr int KT_STEP = SPLIT ? kWaves32 : 1;

    if (kt_first < kt_end) {
        load_tile(kt_first);
        store_tile(0);
    }
    if (!SPLIT) __syncthreads();

    for (int kt = kt_first; kt < kt_end; kt += KT_STEP) {
        const int buf = SPLIT ? 0 : (kt - kt_begin) & 1;
        const bool has_next = kt + KT_STEP < kt_end;
        if (has_next) load_tile(kt + KT_STEP);

        const int k0 = kt * BN;
        const int cls = classify<MASK>(wrow0, k0, k0 + BN - 1, S, W);
        auto tile_body = [&](auto edge_tag) {
            constexpr bool EDGE = decltype(edge_tag)::value;
            const float *Kf = stage0 + buf * TL::STAGE;
            const float *Vf = Kf + TL::K_ELEMS;

            f32x16 sacc = f32x16{};
#pragma unroll
            for (int s = 0; s < D / 2; ++s) {
                const int d = s % TL::H + 2 * TL::H * (s / TL::H) + TL::H * g;
                const float a = Kf[c32 * TL::K_LD + d];
                const float bq = __uint_as_float(qf[s / 4][s % 4]);
                sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bq, sacc, 0, 0, 0);
            }
            if constexpr (EDGE) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (!visible<MASK>(row, key, S, W)) sacc[r] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
            mx = half_max(mx);
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * sl2e;
            if (wave_any(mt > m_run + kRescaleLog2)) {
                const float m_new = fmaxf(m_run, mt);
                const float alpha = (m_run == -INFINITY) ? 0.0f : exp2_fast(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int t = 0; t < ND; ++t) oacc[t] *= alpha;
                m_run = m_new;
            }
            const float base = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = exp2_fast(fmaf(sacc[r], sl2e, -base));
                if (EDGE && sacc[r] == -INFINITY) e = 0.0f;
                sacc[r] = e;
                l_run += e;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
                for (int t = 0; t < ND; ++t) {
                    const float a = Vf[key * TL::V_LD + 32 * t + c32];
                    oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[r], oacc[t], 0, 0, 0);
                }
            }
        };
        if (cls == kFull) tile_body(std::false_type{});
        else if (cls == kEdge) tile_body(std::true_type{});

        if constexpr (SPLIT) {
            // The wave's own block: its reads of this tile are issued before
            // the writes of the next one, and LDS executes a wave's
            // operations in order.
            if (has_next) store_tile(0);
        } else {
            if (has_next) store_tile(buf ^ 1);
            __syncthreads();
        }
    }

    if constexpr (SPLIT) {
        // Merge the four waves' (m, l, O): waves 1-3 publish theirs through
        // LDS (same lane layout), wave 0 combines and stores.
        __syncthreads();  // every wave is done with its staging block
        constexpr int PART = 2 + 16 * ND;  // floats per lane
        if (wave > 0) {
            float *part = lds + (wave - 1) * PART * 64;
            part[lane] = m_run;
            part[64 + lane] = l_run;
#pragma unroll
            for (int t = 0; t < ND; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[(2 + 16 * t + r) * 64 + lane] = oacc[t][r];
        }
        __syncthreads();
        if (wave > 0) return;
        float mw[kWaves32];
        mw[0] = m_run;
        float mx = m_run;
#pragma unroll
        for (int w = 1; w < kWaves32; ++w) {
            mw[w] = lds[(w - 1) * PART * 64 + lane];
            mx = fmaxf(mx, mw[w]);
        }
        float f[kWaves32];
#pragma unroll
        for (int w = 0; w < kWaves32; ++w) f[w] = mw[w] == -INFINITY ? 0.0f : exp2_fast(mw[w] - mx);
        l_run *= f[0];
#pragma unroll
        for (int t = 0; t < ND; ++t) oacc[t] *= f[0];
#pragma unroll
        for (int w = 1; w < kWaves32; ++w) {
            const float *pw = lds + (w - 1) * PART * 64;
            l_run += f[w] * pw[64 + lane];
#pragma unroll
            for (int t = 0; t < ND; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[t][r] += f[w] * pw[(2 + 16 * t + r) * 64 + lane];
        }
    }

    const float inv = 1.0f / half_sum(l_run);
    if (row < S) {
        float *orow = O + ((int64_t)b * S + row) * q_row_stride + (int64_t)h * D;
#pragma unroll
        for (int t = 0; t < ND; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 w = {oacc[t][4 * i] * inv, oacc[t][4 * i + 1] * inv, oacc[t][4 * i + 2] * inv,
                           oacc[t][4 * i + 3] * inv};
                *reinterpret_cast<f32x4 *>(orow + 32 * t + 8 * i + 4 * g) = w;
            }
    }
}

}  // namespace fa355
