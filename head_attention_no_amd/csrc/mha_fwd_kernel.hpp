// Fused no-KV-cache multi-head attention forward for gfx950 (MI355X).
//
// Computes answer = softmax(mask(scale * Q K^T)) V per (batch, head), the
// operator of the "FlashAttentionGPU" API page (max.modular.com, section
// "execute", Steps 0-4), with the online-softmax (FlashAttention-2)
// reduction over key tiles described on the recipe page "Custom Operations:
// Applications in AI Models" (section "Optimizing attention via
// FlashAttention") and in tiny_flash_attn.py's flash_attn_v2: running row
// max m and row sum l, output rescaled by exp(m_old - m_new), divided by l
// once after the last key tile.
//
// Decomposition: one 256-thread workgroup (4 waves of 64 lanes) per
// (query tile of 128 rows, batch b, head h); each wave owns 32 query rows.
//
// Register layouts (32x32 MFMA, lane = 0..63, c = lane % 32, g = lane / 32):
//  * Scores are computed transposed, S^T = K Q^T, so that the accumulator
//    column is the query row: lane (c, g) holds, for key sub-tile t,
//    S^T[key = 32t + 8i + 4g + j][query = c] in element 4i + j. A query row
//    therefore lives in two lanes (c and c + 32); its max and sum need one
//    cross-half exchange (v_permlane32_swap) per key tile.
//  * Q is the B operand and stays in registers for the whole key loop.
//  * The probabilities P^T are used in place as the B operand of
//    O^T = V^T P^T: for PV step s the 8 values are accumulator elements
//    8(s%2) .. 8(s%2)+7 of sub-tile s/2, i.e. keys 16s + 8(e/4) + 4g + e%4.
//    V^T is staged in LDS with the key order permuted to match, so no
//    register shuffle is needed between the two products.
//  * O^T accumulates in fp32: lane (c, g) holds O[query c][d = 32t + 8i + 4g + j].
//
// LDS: two stages (double buffering) of {K tile [BN][D], V^T tile [D][BN]}
// with rows padded by 16 bytes so that 16-byte reads of 32 consecutive rows
// and the transposing 16-byte writes hit distinct banks.
//
// Masking: key tiles wholly hidden from a wave are skipped (the workgroup
// only loads tiles that some of its rows can see); tiles wholly visible run
// without any per-element test; only edge tiles (the diagonal, the window's
// far edge, the ragged end of the sequence) test each element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };

// Kernel arguments (one struct, passed by value).
struct Params {
    void *out;
    const void *q;
    const void *k;
    const void *v;
    int B, S, H, Hkv;
    int rep;       // H / Hkv: query heads per K/V head
    int n_qtiles;  // ceil(S / BM)
    int window;    // sliding-window width, clamped to S (a window >= S is causal)
    float scale_log2;  // |scale| * log2(e): exp(scale*s) = exp2(s * scale_log2) for scale >= 0
    uint32_t q_sign;   // sign-bit mask XORed into Q so that scale < 0 becomes |scale|
};

constexpr int kThreads = 256;  // 4 waves
constexpr int kBlockM = 128;   // query rows per workgroup (32 per wave)

// Lazy rescaling: the running max is only raised when a new tile's max
// exceeds it by more than this many powers of two, so P stays <= 2^8 and
// most tiles skip the O rescale altogether.
constexpr float kRescaleLog2 = 8.0f;

template <typename T, int D>
struct Tile {
    static constexpr bool k16 = sizeof(T) == 2;
    static constexpr int BN = k16 ? 8192 / D : 32;  // keys per tile
    static constexpr int NKT = BN / 32;              // 32-key sub-tiles of S^T
    static constexpr int ND = D / 32;                // 32-dim sub-tiles of O^T
    // LDS row strides in elements: 16-byte padding for 16-bit types; for
    // fp32, K rows are padded by one float (odd stride) and V rows by 8.
    static constexpr int K_LD = k16 ? D + 8 : D + 1;
    static constexpr int V_LD = k16 ? BN + 8 : D + 8;
    static constexpr int K_ELEMS = BN * K_LD;
    static constexpr int V_ELEMS = k16 ? D * V_LD : BN * V_LD;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * (int)sizeof(T);
    static_assert(D == 64 || D == 128, "head dim");
};

// Workgroup -> (query tile, batch, head). Hardware dispatches workgroup w to
// XCD w % 8 as that XCD's (w / 8)-th workgroup. When the (batch, K/V head)
// groups split evenly over the 8 XCDs, every XCD gets whole groups (so the
// H/Hkv query heads that share K/V also share that XCD's L2) and the same
// mix of tile lengths; within an XCD, and in the fallback order, the longest
// query tiles (the last ones, under a causal mask) start first.
struct TileCoord {
    int qt, b, h;
};

__host__ __device__ inline TileCoord block_coord(int w, int n_qtiles, int B, int H, int Hkv)
{
    const int rep = H / Hkv;
    const int groups = B * Hkv;
    TileCoord c;
    if (groups % 8 == 0) {
        const int x = w % 8, slot = w / 8;
        const int per_tile = (groups / 8) * rep;
        const int qi = slot / per_tile;
        const int rem = slot % per_tile;
        const int grp = (rem / rep) * 8 + x;
        c.b = grp / Hkv;
        c.h = (grp % Hkv) * rep + rem % rep;
        c.qt = n_qtiles - 1 - qi;
    } else {
        const int bh = B * H;
        c.qt = n_qtiles - 1 - w / bh;
        c.b = (w % bh) / H;
        c.h = w % H;
    }
    return c;
}

// ---------------------------------------------------------------------------
// device helpers

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value with the one held by lane ^ 32 (the other half of
// the same query row): returns op(x[lane], x[lane ^ 32]) in every lane.
__device__ inline float half_max(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ inline float half_sum(float x)
{
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ inline bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Round 2 floats to a packed pair of 16-bit values (round to nearest even).
template <typename T>
__device__ inline uint32_t pack2(float a, float b);

template <>
__device__ inline uint32_t pack2<__bf16>(float a, float b)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

template <>
__device__ inline uint32_t pack2<_Float16>(float a, float b)
{
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f32x2 f = {a, b};
    f16x2 h = __builtin_convertvector(f, f16x2);
    return __builtin_bit_cast(uint32_t, h);
}

template <typename T>
__device__ inline f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ inline f32x16 mfma16<__bf16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <>
__device__ inline f32x16 mfma16<_Float16>(u32x4 a, u32x4 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Tile classification for one wave's 32 rows [r0, r0+31] and keys [k0, k1].
enum TileClass { kEmpty = 0, kFull = 1, kEdge = 2 };

template <int MASK>
__device__ inline int classify(int r0, int k0, int k1, int S, int W)
{
    if (r0 >= S) return kEmpty;  // padding rows only
    const int r1 = r0 + 31;
    const bool tail = k1 >= S;
    if (MASK == kMaskNone) return tail ? kEdge : kFull;
    if (k0 > r1) return kEmpty;
    if (MASK == kMaskWindow && k1 <= r0 - W) return kEmpty;
    bool full = k1 <= r0 && !tail;
    if (MASK == kMaskWindow) full = full && k0 > r1 - W;
    return full ? kFull : kEdge;
}

template <int MASK>
__device__ inline bool visible(int row, int key, int S, int W)
{
    if (key >= S) return false;
    if (MASK == kMaskNone) return true;
    if (key > row) return false;
    if (MASK == kMaskWindow) return key > row - W;
    return true;
}

// ---------------------------------------------------------------------------
// The kernel.

template <typename T, int D, int MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mha_fwd(Params p)
{
    using TL = Tile<T, D>;
    constexpr bool k16 = TL::k16;
    constexpr int BN = TL::BN;
    constexpr int NKT = TL::NKT;
    constexpr int ND = TL::ND;

    __shared__ __attribute__((aligned(16))) T lds[2 * TL::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c32 = lane & 31;
    const int g = lane >> 5;

    const TileCoord tc = block_coord(blockIdx.x, p.n_qtiles, p.B, p.H, p.Hkv);
    const int b = tc.b, h = tc.h, kvh = h / p.rep;
    const int S = p.S, W = p.window;
    const int q0 = tc.qt * kBlockM;
    const int wrow0 = q0 + wave * 32;
    const int row = wrow0 + c32;  // this lane's query row

    const T *__restrict__ Q = static_cast<const T *>(p.q);
    const T *__restrict__ K = static_cast<const T *>(p.k);
    const T *__restrict__ V = static_cast<const T *>(p.v);
    T *__restrict__ O = static_cast<T *>(p.out);

    const int64_t q_row_stride = (int64_t)p.H * D;
    const int64_t kv_row_stride = (int64_t)p.Hkv * D;
    const T *Kbh = K + (int64_t)b * S * kv_row_stride + (int64_t)kvh * D;
    const T *Vbh = V + (int64_t)b * S * kv_row_stride + (int64_t)kvh * D;

    // ---- Q fragments (B operand), loaded once ----------------------------
    // 16-bit: qf[s] = Q[row][16s + 8g .. +7]. fp32: element s of lane group
    // g is Q[row][dsel(s, g)], dsel(s,g) = (s%32) + 64(s/32) + 32g.
    constexpr int NQ = k16 ? D / 16 : D / 8;  // 16-byte registers
    u32x4 qf[NQ];
    {
        const T *qrow = Q + ((int64_t)b * S + row) * q_row_stride + (int64_t)h * D;
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            int d;
            if constexpr (k16) d = 16 * s + 8 * g;
            else d = (4 * s) % 32 + 64 * ((4 * s) / 32) + 32 * g;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row < S) x = ldg16(qrow + d);
            x ^= p.q_sign;
            qf[s] = x;
        }
    }

    // ---- key-tile range of this workgroup ---------------------------------
    const int q_last = min(q0 + kBlockM, S) - 1;
    int kt_begin = 0;
    int kt_end = (S + BN - 1) / BN;
    if (MASK != kMaskNone) kt_end = min(kt_end, q_last / BN + 1);
    if (MASK == kMaskWindow) kt_begin = max(0, q0 - W + 1) / BN;

    // ---- staging of one K/V tile: global -> registers -> LDS -------------
    // 16-bit: waves 0-1 stage V^T (8 keys x 8 dims per thread, transposed in
    // registers), waves 2-3 stage K (8 rows x 16 bytes per thread).
    // fp32: every thread stages D/32 rows of K and of V (16 bytes each).
    constexpr int NSTG = k16 ? 8 : 2 * (D / 32);
    u32x4 stg[NSTG];

    auto load_tile = [&](int kt) {
        const int k0 = kt * BN;
        if constexpr (k16) {
            if (wave < 2) {
                const int t = tid;                 // 0..127
                const int ks = t % (BN / 8);       // key set: 16(ks/2) + 4(ks%2) + {0..3, 8..11}
                const int c = t / (BN / 8);        // 8-dim chunk
                const int kbase = k0 + 16 * (ks >> 1) + 4 * (ks & 1);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int key = kbase + 8 * (r >> 2) + (r & 3);
                    u32x4 x = {0u, 0u, 0u, 0u};
                    if (key < S) x = ldg16(Vbh + (int64_t)key * kv_row_stride + 8 * c);
                    stg[r] = x;
                }
            } else {
                const int t = tid - 128;
                constexpr int CPR = D / 8;         // 16-byte chunks per row
                constexpr int STEP = 128 / CPR;
                const int c = t % CPR, kr = t / CPR;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int key = k0 + kr + r * STEP;
                    u32x4 x = {0u, 0u, 0u, 0u};
                    if (key < S) x = ldg16(Kbh + (int64_t)key * kv_row_stride + 8 * c);
                    stg[r] = x;
                }
            }
        } else {
            constexpr int CPR = D / 4;
            constexpr int STEP = kThreads / CPR;
            constexpr int R = BN / STEP;
            const int c = tid % CPR, kr = tid / CPR;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int key = k0 + kr + r * STEP;
                u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
                if (key < S) {
                    xk = ldg16(Kbh + (int64_t)key * kv_row_stride + 4 * c);
                    xv = ldg16(Vbh + (int64_t)key * kv_row_stride + 4 * c);
                }
                stg[r] = xk;
                stg[R + r] = xv;
            }
        }
    };

    auto store_tile = [&](int buf) {
        T *Ks = lds + buf * TL::STAGE;
        T *Vs = Ks + TL::K_ELEMS;
        if constexpr (k16) {
            if (wave < 2) {
                const int t = tid;
                const int ks = t % (BN / 8);
                const int c = t / (BN / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // Row d = 8c + e of V^T: the 8 keys of this set, slot order.
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    const int w = e >> 1;
                    u32x4 o;
                    o[0] = __builtin_amdgcn_perm(stg[1][w], stg[0][w], sel);
                    o[1] = __builtin_amdgcn_perm(stg[3][w], stg[2][w], sel);
                    o[2] = __builtin_amdgcn_perm(stg[5][w], stg[4][w], sel);
                    o[3] = __builtin_amdgcn_perm(stg[7][w], stg[6][w], sel);
                    *reinterpret_cast<u32x4 *>(Vs + (8 * c + e) * TL::V_LD + 8 * ks) = o;
                }
            } else {
                const int t = tid - 128;
                constexpr int CPR = D / 8;
                constexpr int STEP = 128 / CPR;
                const int c = t % CPR, kr = t / CPR;
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    *reinterpret_cast<u32x4 *>(Ks + (kr + r * STEP) * TL::K_LD + 8 * c) = stg[r];
            }
        } else {
            constexpr int CPR = D / 4;
            constexpr int STEP = kThreads / CPR;
            constexpr int R = BN / STEP;
            const int c = tid % CPR, kr = tid / CPR;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int key = kr + r * STEP;
                float *kd = reinterpret_cast<float *>(Ks) + key * TL::K_LD + 4 * c;
#pragma unroll
                for (int e = 0; e < 4; ++e) kd[e] = __uint_as_float(stg[r][e]);
                *reinterpret_cast<u32x4 *>(reinterpret_cast<float *>(Vs) + key * TL::V_LD + 4 * c) =
                    stg[R + r];
            }
        }
    };

    // ---- running state ----------------------------------------------------
    f32x16 oacc[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) oacc[t] = f32x16{};
    float m_run = -INFINITY;  // running max, in scaled log2 units
    float l_run = 0.0f;       // this lane's share of the running sum
    const float sl2e = p.scale_log2;

    load_tile(kt_begin);
    store_tile(0);
    __syncthreads();

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        const bool has_next = kt + 1 < kt_end;
        if (has_next) load_tile(kt + 1);

        const int k0 = kt * BN;
        const int cls = classify<MASK>(wrow0, k0, k0 + BN - 1, S, W);
        if (cls != kEmpty) {
            const T *Ks = lds + buf * TL::STAGE;
            const T *Vs = Ks + TL::K_ELEMS;

            // S^T = K Q^T for this tile.
            f32x16 sacc[NKT];
#pragma unroll
            for (int t = 0; t < NKT; ++t) sacc[t] = f32x16{};
            if constexpr (k16) {
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
#pragma unroll
                    for (int t = 0; t < NKT; ++t) {
                        const u32x4 a = *reinterpret_cast<const u32x4 *>(
                            Ks + (32 * t + c32) * TL::K_LD + 16 * s + 8 * g);
                        sacc[t] = mfma16<T>(a, qf[s], sacc[t]);
                    }
                }
            } else {
                const float *Kf = reinterpret_cast<const float *>(Ks);
#pragma unroll
                for (int s = 0; s < D / 2; ++s) {
                    const int d = (s % 32) + 64 * (s / 32) + 32 * g;
                    const float a = Kf[c32 * TL::K_LD + d];
                    const float bq = __uint_as_float(qf[s / 4][s % 4]);
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bq, sacc[0], 0, 0, 0);
                }
            }

            // Mask, online softmax.
            if (cls == kEdge) {
#pragma unroll
                for (int t = 0; t < NKT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
                        if (!visible<MASK>(row, key, S, W)) sacc[t][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
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
            float psum = 0.0f;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float e = exp2_fast(fmaf(sacc[t][r], sl2e, -base));
                    if (cls == kEdge && sacc[t][r] == -INFINITY) e = 0.0f;
                    sacc[t][r] = e;
                    psum += e;
                }
            l_run += psum;

            // O^T += V^T P^T.
            if constexpr (k16) {
#pragma unroll
                for (int s = 0; s < BN / 16; ++s) {
                    const f32x16 &pt = sacc[s >> 1];
                    const int o8 = 8 * (s & 1);
                    u32x4 pb;
                    pb[0] = pack2<T>(pt[o8 + 0], pt[o8 + 1]);
                    pb[1] = pack2<T>(pt[o8 + 2], pt[o8 + 3]);
                    pb[2] = pack2<T>(pt[o8 + 4], pt[o8 + 5]);
                    pb[3] = pack2<T>(pt[o8 + 6], pt[o8 + 7]);
#pragma unroll
                    for (int t = 0; t < ND; ++t) {
                        const u32x4 a = *reinterpret_cast<const u32x4 *>(
                            Vs + (32 * t + c32) * TL::V_LD + 16 * s + 8 * g);
                        oacc[t] = mfma16<T>(a, pb, oacc[t]);
                    }
                }
            } else {
                const float *Vf = reinterpret_cast<const float *>(Vs);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 8 * (r >> 2) + 4 * g + (r & 3);
#pragma unroll
                    for (int t = 0; t < ND; ++t) {
                        const float a = Vf[key * TL::V_LD + 32 * t + c32];
                        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[0][r], oacc[t], 0, 0, 0);
                    }
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l, written back in BSHD -----------------------
    const float l_tot = half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (row < S) {
        T *orow = O + ((int64_t)b * S + row) * q_row_stride + (int64_t)h * D;
#pragma unroll
        for (int t = 0; t < ND; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 32 * t + 8 * i + 4 * g;
                const float x0 = oacc[t][4 * i + 0] * inv, x1 = oacc[t][4 * i + 1] * inv;
                const float x2 = oacc[t][4 * i + 2] * inv, x3 = oacc[t][4 * i + 3] * inv;
                if constexpr (k16) {
                    u32x2 w = {pack2<T>(x0, x1), pack2<T>(x2, x3)};
                    *reinterpret_cast<u32x2 *>(orow + d) = w;
                } else {
                    f32x4 w = {x0, x1, x2, x3};
                    *reinterpret_cast<f32x4 *>(orow + d) = w;
                }
            }
    }
}

}  // namespace fa355
