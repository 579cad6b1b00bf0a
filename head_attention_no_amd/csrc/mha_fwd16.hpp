// bf16 / fp16 attention forward for gfx950 (MI355X).
//
// Online-softmax (FlashAttention-2) reduction over key tiles: the
// "Optimizing attention via FlashAttention" section of the recipe page
// "Custom Operations: Applications in AI Models" and tiny_flash_attn.py's
// flash_attn_v2 keep a running row max m and row sum l per query, rescale
// the output by exp(m_old - m_new) and divide by l once after the last key
// tile. Scale and mask are applied to the scores before the softmax, as the
// "FlashAttentionGPU" API page (section "execute", Step 3) specifies.
//
// Decomposition: one workgroup of NW waves (8, or 4 at D = 256) per
// (query tile, batch, group of hp heads sharing a K/V head); each wave owns
// 32 query rows of one head, so a query tile is 32 NW / hp rows; key tiles
// of BN keys (Tile16 below).
//
// Register layouts (32x32x16 MFMA; lane = 0..63, c = lane % 32, g = lane / 32):
//  * Scores are computed transposed, S^T = K Q^T, so the accumulator column
//    is the query row: lane (c, g) holds, for 32-key sub-tile t,
//    S^T[key = 32t + 8i + 4g + j][query c] in element 4i + j. A query row
//    lives in two lanes (c and c + 32); its max needs one v_permlane32_swap
//    per key tile and its sum one at the very end.
//  * Q is the B operand (k-step s: Q[c][16s + 8g .. +7]) and stays in
//    registers for the whole key loop.
//  * P^T is used in place as the B operand of O^T = V^T P^T: for PV k-step
//    s the 8 values are accumulator elements 8(s%2) .. 8(s%2)+7 of sub-tile
//    s/2, i.e. keys 16s + 8(e/4) + 4g + e%4 (e = 0..7). The V^T A operand is
//    read with the transposing LDS load ds_read_b64_tr_b16, two per
//    operand, which delivers exactly that key order (see below).
//  * O^T accumulates in fp32: lane (c, g) holds O[query c][d = 32t + 8i + 4g + j].
//
// K/V staging: buffer_load_dwordx4 ... lds copies 16-byte pieces straight
// from global memory into LDS (lane l of a copy lands at byte 16 l of a
// 1 KiB block), double buffered, with no register staging. A 1 KiB block
// holds one key group of G = 512 / D keys (4 or 8) in full, as 16-byte
// slots ordered [chunk][key in group]:
//    K: slot = (chunk ^ swK(group)) * G + key%G
//    V: slot = chunk * G + (key%G ^ swV(chunk))
// The XOR swizzles make the 16 lanes that share a bank cycle read distinct
// banks, and keep every read address of a tile an immediate offset from one
// per-lane base. Rows past the end of the sequence fall outside the buffer
// resource's range and read as zero.
//
// ds_read_b64_tr_b16, per 16-lane group: lane i receives element i%4 of the
// 8 bytes addressed by lane 4k + i/4, for k = 0..3. Lane 16q + j addresses
// V[key 4(q/2) + j/4 (+16s, +8 for the second half)][d 16(q%2) + 4(j%4)
// (+32t) .. +3], so lane (c, g) receives V[16s + 4g + k (+8)][32t + c].
//
// Masking: key tiles wholly hidden from a wave are skipped (the workgroup
// only copies tiles some of its rows can see); tiles wholly visible run
// without any per-element test; only edge tiles (the diagonal, the window's
// far edge, the ragged end of the sequence) test each element.
#pragma once

#include "mha_common.hpp"

namespace fa355 {

// Word 3 of a raw buffer resource (untyped 32-bit access, range checked).
constexpr int kRsrcWord3 = 0x00020000;

// Per head dim D: keys per tile BN (S^T tiles and the V steps in flight fit
// the registers), waves per workgroup NW and waves per SIMD WPE, and the LDS
// swizzle periods (below).
// D = 256 has two layouts. The default one, like D = 128, runs 8 waves of
// 32 rows, two per SIMD, with 32-key tiles: the Q fragments and O^T take 192
// of a wave's 256 registers, and the 16 scores and the operands in flight
// fit the rest. FEW (chosen by the host for calls with few work items, see
// layout_of in fa355.hip) runs 4 waves, one per SIMD, with 64-key tiles and
// the pipelined loop: half the rows per work item, so twice the items, which
// balances causal calls of under two 256-row items per compute unit; there
// the compiler keeps S^T and O^T in the accumulation registers and moves
// O^T out to vector registers on every tile, which the default layout
// (no accumulation registers) avoids: 6-20 % faster where items suffice.
template <int D, bool FEW = false>
struct Tile16 {
    static_assert(!FEW || D == 256, "the few-item layout exists at D = 256 only");
    static constexpr int BN = D == 32 ? 128 : (D == 256 && !FEW) ? 32 : 64;  // keys per tile
    static constexpr int NW = FEW ? 4 : 8;           // waves per workgroup, 32 query rows each
    // Waves per SIMD: D = 32 and 64, bound by the vector units and at 120
    // registers (64-key tiles at D = 64), run two workgroups per CU (4 waves
    // per SIMD: 8-20 % faster than 2 at D = 32, 3-7 % at D = 64).
    static constexpr int WPE = FEW ? 1 : D <= 64 ? 4 : 2;
    static constexpr int NKT = BN / 32;           // 32-key sub-tiles of S^T
    static constexpr int ND = D / 32;             // 32-dim sub-tiles of O^T
    static constexpr int G = 512 / D;             // keys per 1 KiB key group
    static constexpr int TILE_BYTES = BN * D * 2;  // 8, 16 or 32 KiB
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile, then V tile
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;   // double buffered
    static constexpr int GROUPS = BN / G;         // key groups per tile
    static constexpr int KP = D == 256 ? 4 : D == 128 ? 2 : 1;  // K read address bases
    static constexpr int VT = D == 256 ? 2 : 1;   // V read bases per 32-dim sub-tile period
    static constexpr int VH = D == 32 ? 2 : 1;    // V read bases per 8-key half period
    static constexpr int V_AHEAD = 2 * ND <= 8 ? 2 : 1;  // PV k-steps whose V reads are in flight
    // Plain loop at D = 128 and 256: V reads issued per PV MFMA, this many
    // MFMAs ahead, instead of per k-step (0). At D = 256 a k-step's 16 reads
    // would take 32 registers (the kernel then spills); at D = 128 it frees
    // 12 registers and was 0.5-1.3 % faster on four of five shapes.
    static constexpr int V_PAIRS_AHEAD = (D == 256 && !FEW) || D == 128 ? 4 : 0;
    // Software-pipelined key loop (the next tile's S MFMAs interleaved with
    // this tile's softmax, then its PV MFMAs with the next tile's max), in an
    // issue order fixed at compile time: used by the few-item layout at
    // D = 256, where one wave per SIMD leaves no second wave to hide the
    // softmax (17 % faster there than the plain loop in that layout). The
    // plain loop, with its counted K reads, is as fast or faster at D = 64
    // (level unmasked, 1.6 %-5 % faster causal and windowed), and faster at
    // D = 32 (bound by the vector units) and D = 128 (held at the power cap,
    // where the extra S MFMAs of each wave's last tile cost more than the
    // overlap gains).
    static constexpr bool PIPELINE = FEW;
    // The plain loop can walk several work items per workgroup (prefetching
    // the next item's Q rows and first K/V tile); calls use that at D = 64
    // and 128 (walks() in mha_common.hpp).
    static constexpr bool WALK = D == 64 || D == 128;
    // At D = 32 and 64, bound by the vector units, Q can be scaled by
    // scale * log2(e) once per work item (rounded to T) with each tile's
    // score accumulators starting at -m, so the MFMA result is already the
    // exponent s * scale * log2(e) - m and the per-score fma disappears
    // (10 % faster on the unmasked fp16 S = 16384 workload; at D = 128 it
    // saved 1 % and is not built). The rounding of the scaled Q changes
    // each product of the exponent by at most half a unit in the last place
    // of T. The launcher uses it unless the scaled Q could leave fp16's
    // range (|scale| log2(e) > 1 with fp16 inputs).
    static constexpr bool PRESCALE = D <= 64;
    static constexpr int PIPE_K_AHEAD = 3;    // K operand reads issued this many MFMAs ahead
    static constexpr int PIPE_V_AHEAD = 4;    // V operand pairs issued this many MFMAs ahead
    static constexpr int PIPE_MAX_DELAY = 3;  // MFMAs between the last S MFMA and its max
    static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dim");
    static_assert(GROUPS % NW == 0, "every wave copies the same number of key groups");
};

// XOR swizzles of the 1 KiB key-group blocks (kg = key / G, ks = key % G,
// c = 16-byte chunk of the row): K slot (c ^ k_swz(kg)) G + ks, V slot
// (c ^ vc_swz(kg)) G + (ks ^ vk_swz(c)). They make the 16 lanes of a K read
// cycle, and the 32 lanes of a V read cycle, hit 64 distinct banks.
template <int D>
__device__ inline int k_swz(int kg) { return kg & (D / 32 - 1); }
template <int D>
__device__ inline int vc_swz(int kg) { return D == 256 ? 4 * (kg & 1) : 0; }
template <int D>
__device__ inline int vk_swz(int c)
{
    return D == 32 ? (4 * ((c >> 1) & 1)) ^ (8 * (c & 1)) : D == 64 ? 4 * ((c >> 1) & 1) : 0;
}

// Byte offsets of K[key][16-byte chunk c] and V[key][c] inside a tile region.
template <int D>
__device__ inline int k_lds_offset(int key, int c)
{
    constexpr int G = Tile16<D>::G;
    const int kg = key / G;
    return kg * 1024 + ((c ^ k_swz<D>(kg)) * G + key % G) * 16;
}
template <int D>
__device__ inline int v_lds_offset(int key, int c)
{
    constexpr int G = Tile16<D>::G;
    const int kg = key / G;
    return kg * 1024 + ((c ^ vc_swz<D>(kg)) * G + ((key % G) ^ vk_swz<D>(c))) * 16;
}

// Transposing LDS read at byte address addr + OFF (see the layout note above).
// Written as inline asm: the compiler cannot tell this read apart from the
// in-flight global -> LDS copies of the next tile and would otherwise wait
// for them before every such read. The ordering it would enforce is already
// explicit (copies are waited for and barriered before a tile is read), so
// only the read's own completion is needed: lds_wait() below.
template <int OFF>
__device__ inline u32x2 lds_read_tr16(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset field");
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}

// Wait until at most PENDING of this wave's LDS operations are outstanding
// (LDS operations complete in issue order, so every read issued before the
// PENDING most recent ones has returned), and make the registers in `r`
// depend on that wait. PENDING counts only reads issued after those in `r`;
// anything else issued later only makes the wait stricter.
template <int PENDING, int N>
__device__ inline void lds_wait(u32x2 (&r)[N])
{
    static_assert(PENDING >= 0 && PENDING <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(PENDING) : "memory");
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(r[i]));
}

// Make r depend on the last wait (for reads waited for by an earlier lds_wait).
__device__ inline void lds_tie(u32x2 &r) { asm volatile("" : "+v"(r)); }

// 16-byte LDS read at byte address addr + OFF, as inline asm for the same
// reason as lds_read_tr16, waited for with lds_wait4().
template <int OFF>
__device__ inline u32x4 lds_read_b128(uint32_t addr)
{
    static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset field");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
    return r;
}

template <int PENDING>
__device__ inline void lds_wait4(u32x4 &r)
{
    static_assert(PENDING >= 0 && PENDING <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(PENDING) : "memory");
    asm volatile("" : "+v"(r));
}

__device__ inline void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, uint8_t *lds_dst, uint32_t voffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_dst,
                                             16, voffset, 0, 0, 0);
}

// Wait for this wave's outstanding global -> LDS copies (vmcnt = 0).
__device__ inline void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// q * c for the 8 16-bit values of a Q fragment, rounded to T (nearest even).
template <typename T>
__device__ inline u32x4 scale_frag(u32x4 x, float c);

template <>
__device__ inline u32x4 scale_frag<__bf16>(u32x4 x, float c)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(x[i] << 16), hi = __uint_as_float(x[i] & 0xFFFF0000u);
        r[i] = pack2<__bf16>(lo * c, hi * c);
    }
    return r;
}

template <>
__device__ inline u32x4 scale_frag<_Float16>(u32x4 x, float c)
{
    // The halves go through 16-bit integers: a bit_cast of the vector
    // element to a half pair inside this loop compiled to element 0 only.
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = x[i];
        const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
        const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
        r[i] = pack2<_Float16>((float)lo * c, (float)hi * c);
    }
    return r;
}

// One work item (a query tile of hp heads sharing a K/V head) as one wave
// of the workgroup sees it.
struct WaveItem {
    int b, kvh, h;           // batch, K/V head, this wave's query head
    int q0, wrow0, row;      // first row of the tile, of this wave, of this lane
    int kt_begin, kt_end;    // key tiles the workgroup visits
    int64_t kv_head0;        // byte offset of K/V[b, 0, kvh, 0]
};

template <int D, int MASK, int BN>
__device__ inline WaveItem wave_item(const Params &p, int item, int wave, int c32)
{
    const TileCoord tc = block_coord(item, p.n_qtiles, p.B, p.H, p.Hkv, p.hp, p.group_order);
    const int rows = 32 * p.wph;  // query rows per head in the workgroup
    WaveItem it;
    it.b = tc.b;
    it.kvh = tc.h / p.rep;
    it.h = tc.h + wave / p.wph;
    it.q0 = tc.qt * rows;
    it.wrow0 = it.q0 + (wave % p.wph) * 32;
    it.row = it.wrow0 + c32;
    it.kv_head0 = ((int64_t)it.b * p.S * p.Hkv + it.kvh) * D * 2;
    key_tile_range<MASK, BN>(it.q0, rows, p.S, p.window, it.kt_begin, it.kt_end);
    return it;
}

// Tile16<D, FEW>::NW waves per workgroup, 32 query rows each.
// PRE: the pre-scaled Q (Tile16<D>::PRESCALE) of the plain loop; FEW: the
// few-item layout at D = 256.
template <typename T, int D, int MASK, bool PRE, bool FEW = false>
__global__ __launch_bounds__((64 * Tile16<D, FEW>::NW))
__attribute__((amdgpu_waves_per_eu((Tile16<D, FEW>::WPE), (Tile16<D, FEW>::WPE))))
void mha_fwd16(Params p)
{
    using TL = Tile16<D, FEW>;
    static_assert(!PRE || (TL::PRESCALE && !TL::PIPELINE), "pre-scaled Q: plain loop, D <= 64");
    constexpr int NW = TL::NW;
    constexpr int NTHREADS = 64 * NW;
    constexpr int NCOPY = TL::GROUPS / NW;  // key groups of K (and of V) each wave copies per tile
    constexpr int KP = TL::KP, VT = TL::VT, VH = TL::VH, V_AHEAD = TL::V_AHEAD;
    constexpr int BN = TL::BN;
    constexpr int NKT = TL::NKT;
    constexpr int ND = TL::ND;
    constexpr int G = TL::G;

    // K/V stages, then (plain loop only) each wave's 32 Q rows of the next
    // work item: D / 16 blocks of 1 KiB, lane l's 16 bytes of k-step s at
    // block s, byte 16 l.
    constexpr int Q_LDS_BYTES = TL::WALK ? NW * D * 64 : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[TL::LDS_BYTES + Q_LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int c32 = lane & 31;
    const int g = lane >> 5;

    const WaveItem it0 = wave_item<D, MASK, BN>(p, blockIdx.x, wave, c32);
    const int S = p.S, W = p.window;
    const int wrow0 = it0.wrow0, row = it0.row;

    T *__restrict__ O = static_cast<T *>(p.out);
    const int64_t q_row_stride = (int64_t)p.H * D;
    const uint32_t kv_stride = (uint32_t)p.Hkv * D * 2;  // bytes between key rows
    const uint8_t *Kbh = static_cast<const uint8_t *>(p.k) + it0.kv_head0;
    const uint8_t *Vbh = static_cast<const uint8_t *>(p.v) + it0.kv_head0;

    // LDS starts zeroed, so a slot no copy writes still holds finite data.
    for (int i = tid; i < TL::LDS_BYTES / 16; i += NTHREADS)
        reinterpret_cast<u32x4 *>(lds)[i] = u32x4{0u, 0u, 0u, 0u};

    // Q fragments: qf[s] = Q[row][16s + 8g .. +7]. Rows past the end of the
    // sequence read the last row (their results are never stored).
    auto load_q = [&](const WaveItem &it, u32x4 (&dst)[D / 16]) {
        const T *qrow = static_cast<const T *>(p.q) + ((int64_t)it.b * S + min(it.row, S - 1)) * q_row_stride +
                        (int64_t)it.h * D;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            dst[s] = ldg16(qrow + 16 * s + 8 * g) ^ p.q_sign;
            if constexpr (PRE) dst[s] = scale_frag<T>(dst[s], p.scale_log2);
        }
    };
    u32x4 qf[D / 16];
    load_q(it0, qf);

    // Copy offsets: wave w copies key groups w, w+NW, ... of K and of V;
    // lane l fills slot l of the group's 1 KiB block.
    uint32_t voff_k[NCOPY], voff_v[NCOPY];
#pragma unroll
    for (int n = 0; n < NCOPY; ++n) {
        const int kg = wave + NW * n;
        const int slot_c = lane / G, slot_k = lane % G;  // lane l fills slot l = slot_c G + slot_k
        voff_k[n] = (kg * G + slot_k) * kv_stride + (slot_c ^ k_swz<D>(kg)) * 16;
        const int vc = slot_c ^ vc_swz<D>(kg);
        voff_v[n] = (kg * G + (slot_k ^ vk_swz<D>(vc))) * kv_stride + vc * 16;
    }
    auto tile_rsrc = [&](const uint8_t *base, int kt) {
        const int k0 = kt * BN;
        // The resource covers the tile's own rows k0 .. min(k0 + BN, S) - 1
        // (at most BN rows, so the range fits 32 bits whatever the size of
        // the tensor); rows past the end of the sequence read as zero.
        const int nrec = (min(BN, S - k0) - 1) * (int)kv_stride + D * 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base) + (int64_t)k0 * kv_stride,
                                                 0, nrec, kRsrcWord3);
    };
    auto copy_tile = [&](const uint8_t *kbase, const uint8_t *vbase, int kt, int stage) {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, kt), rv = tile_rsrc(vbase, kt);
        uint8_t *kdst = lds + stage * TL::STAGE_BYTES;
        uint8_t *vdst = kdst + TL::TILE_BYTES;
#pragma unroll
        for (int n = 0; n < NCOPY; ++n) {
            lds_copy16(rk, kdst + (wave + NW * n) * 1024, voff_k[n]);
            lds_copy16(rv, vdst + (wave + NW * n) * 1024, voff_v[n]);
        }
    };
    auto land_tile = [&](int) { wait_copies(); };

    // Operand read addresses (bytes within a tile region).
    // K: lane (c, g) reads K[32t + c][2s + g] at k_addr[t][s % KP] + (s / KP) 2 KP G 16.
    int k_addr[NKT][KP];
#pragma unroll
    for (int t = 0; t < NKT; ++t)
#pragma unroll
        for (int p = 0; p < KP; ++p) k_addr[t][p] = k_lds_offset<D>(32 * t + c32, 2 * p + g);
    // V (transposing reads): lane 16q + j addresses V[4(q/2) + j/4][16(q%2) + 4(j%4)]
    // plus 16s + 8 half keys and 32t dims: base v_addr[t % VT][half % VH] plus
    // the immediate (16s + 8 (half - half % VH)) / G blocks + (t - t % VT) 64 G bytes.
    const int vq = lane >> 4, vj = lane & 15;
    int v_addr[VT][VH];
#pragma unroll
    for (int tb = 0; tb < VT; ++tb)
#pragma unroll
        for (int hb = 0; hb < VH; ++hb) {
            const int vd = 32 * tb + 16 * (vq & 1) + 4 * (vj & 3);
            v_addr[tb][hb] = v_lds_offset<D>(4 * (vq >> 1) + (vj >> 2) + 8 * hb, vd >> 3) + (vd & 7) * 2;
        }
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)(lds);

    f32x16 oacc[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) oacc[t] = f32x16{};
    float m_run = -INFINITY;  // running max, in scaled log2 units
    float l_run = 0.0f;       // this lane's share of the running sum
    const float sl2e = p.scale_log2;

    const int kt_begin = it0.kt_begin, kt_end = it0.kt_end;

    // Epilogue: O = O^T / l, written back in BSHD with 16-byte stores.
    // Lane (c, g) holds O[c][32t + 8i + 4g .. +3] (4 values, two packed
    // words w[i][0..1]); lanes c and c + 32 swap halves with
    // v_permlane32_swap so that lane g = 0 holds the 8 values of groups
    // i = 0, 1 and lane g = 1 those of i = 2, 3: each lane then stores
    // 16 contiguous bytes per group. The swap exchanges the upper 32 lanes
    // of its first operand with the lower 32 lanes of its second.
    auto store_out = [&](const WaveItem &it) {
        const float inv = 1.0f / half_sum(l_run);
        T *orow = O + ((int64_t)it.b * S + it.row) * q_row_stride + (int64_t)it.h * D;
#pragma unroll
        for (int t = 0; t < ND; ++t) {
            uint32_t w[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    w[i][h] = pack2<T>(oacc[t][4 * i + 2 * h] * inv, oacc[t][4 * i + 2 * h + 1] * inv);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto s0 = __builtin_amdgcn_permlane32_swap(w[i][0], w[i + 2][0], false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(w[i][1], w[i + 2][1], false, false);
                const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
                if (it.row < S) *reinterpret_cast<u32x4 *>(orow + 32 * t + 8 * (i + 2 * g)) = v;
            }
        }
    };

    if constexpr (TL::PIPELINE) {
        constexpr int NPV = BN / 16;    // PV k-steps per tile
        constexpr int NSM = D / 16 * NKT;  // S MFMAs per tile
        constexpr int NPM = NPV * ND;   // PV MFMAs per tile
        constexpr int NM = NSM + NPM;   // MFMAs per step
        constexpr int NPAIR = 4 * NPV;  // score pairs per lane per tile
        constexpr int KA = TL::PIPE_K_AHEAD, VA = TL::PIPE_V_AHEAD, MD = TL::PIPE_MAX_DELAY;

        // Per-lane LDS read bases; the k-step offsets are immediates, and so
        // is the stage offset unless the 16-bit immediate cannot reach the
        // second stage (64 KiB stages at D = 256): then each stage has its
        // own bases.
        constexpr int NB = 2 * TL::STAGE_BYTES > 65536 ? 2 : 1;
        constexpr int IMM_STAGE = NB == 1 ? TL::STAGE_BYTES : 0;
        uint32_t kb[NB][NKT][KP];
        uint32_t vb[NB][VT][VH];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int q = 0; q < KP; ++q) kb[nb][t][q] = lds_base + nb * TL::STAGE_BYTES + k_addr[t][q];
#pragma unroll
            for (int tb = 0; tb < VT; ++tb)
#pragma unroll
                for (int hb = 0; hb < VH; ++hb) vb[nb][tb][hb] = lds_base + nb * TL::STAGE_BYTES + v_addr[tb][hb];
        }

        // K and V of a tile are copied one step apart: K(kt) goes to stage
        // (kt - kt_begin) & 1 one step before V(kt) goes to the same stage.
        auto copy_k = [&](int kt, int stage) {
            const __amdgpu_buffer_rsrc_t rk = tile_rsrc(Kbh, kt);
            uint8_t *kdst = lds + stage * TL::STAGE_BYTES;
#pragma unroll
            for (int n = 0; n < NCOPY; ++n) lds_copy16(rk, kdst + (wave + NW * n) * 1024, voff_k[n]);
        };
        auto copy_v = [&](int kt, int stage) {
            const __amdgpu_buffer_rsrc_t rv = tile_rsrc(Vbh, kt);
            uint8_t *vdst = lds + stage * TL::STAGE_BYTES + TL::TILE_BYTES;
#pragma unroll
            for (int n = 0; n < NCOPY; ++n) lds_copy16(rv, vdst + (wave + NW * n) * 1024, voff_v[n]);
        };
        auto cls_of = [&](int kt) {
            return kt < kt_end ? classify<MASK>(wrow0, kt * BN, kt * BN + BN - 1, S, W) : (int)kEmpty;
        };
        // Element (t, r) holds key k0 + 4g + 32t + 8(r/4) + r%4 (see the
        // plain loop's edge mask).
        auto mask_tile = [&](f32x16 (&sc)[NKT], int k0) {
            int lo, hi;
            visible_range<MASK>(row, k0 + 4 * g, S, W, BN, lo, hi);
            const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 32 * t + 8 * (r >> 2) + (r & 3);
                    const bool vis = MASK == kMaskWindow ? (uint32_t)(off - lo) <= span : off <= hi;
                    if (!vis) sc[t][r] = -INFINITY;
                }
        };
        auto tile_max = [&](f32x16 (&sc)[NKT]) {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
            return half_max(mx) * sl2e;
        };
        // Operand of S MFMA m (k-step m / NKT, sub-tile m % NKT) from stage PAR.
        auto k_read = [&](auto par_tag, auto m_tag) {
            constexpr int PAR = decltype(par_tag)::value, m = decltype(m_tag)::value;
            constexpr int s = m / NKT, t = m % NKT;
            return lds_read_b128<PAR * IMM_STAGE + (s / KP) * 2 * KP * G * 16>(kb[PAR % NB][t][s % KP]);
        };
        // The two transposing reads for PV MFMA j (k-step j / ND, 32-dim sub-tile j % ND) from stage PAR.
        auto v_read = [&](auto par_tag, auto j_tag, u32x2 (&dst)[2]) {
            constexpr int PAR = decltype(par_tag)::value, j = decltype(j_tag)::value;
            constexpr int s = j / ND, t = j % ND;
            constexpr int base = PAR * IMM_STAGE + TL::TILE_BYTES + (t - t % VT) * 64 * G;
            dst[0] = lds_read_tr16<base + (16 * s) / G * 1024>(vb[PAR % NB][t % VT][0]);
            dst[1] = lds_read_tr16<base + (16 * s + 8 * (1 - 1 % VH)) / G * 1024>(vb[PAR % NB][t % VT][1 % VH]);
        };
        // S = K Q^T of the first tile, not interleaved.
        auto s_only = [&](auto par_tag, f32x16 (&sc)[NKT]) {
            constexpr int AH = NSM < 4 ? NSM : 4;  // reads in flight
            u32x4 kr[NSM];
            static_for<AH>([&](auto m_tag) { kr[m_tag] = k_read(par_tag, m_tag); });
            static_for<NSM>([&](auto m_tag) {
                constexpr int m = decltype(m_tag)::value;
                lds_wait4<(m + AH <= NSM ? AH : NSM - m) - 1>(kr[m]);
                sc[m % NKT] = mfma16<T>(kr[m], qf[m / NKT], m < NKT ? f32x16{} : sc[m % NKT]);
                if constexpr (m + AH < NSM) kr[m + AH] = k_read(par_tag, std::integral_constant<int, m + AH>{});
            });
        };

        // Issue plan of one step, fixed at compile time. Slot p holds what is
        // issued right after MFMA p (p = -1: before MFMA 0); MFMAs 0 .. NSM-1 are
        // the next tile's S, then NPM PV MFMAs of this tile.
        //  - K operand m is read in slot m - KA, V operand pair j in slot NSM + j - VA;
        //  - score pair j (fma, exp2, pack, row sum) is computed in slot
        //    j NSM / NPAIR - 1, one per S MFMA at D = 128 and 256, and at the latest
        //    in the slot before the PV MFMAs that consume it;
        //  - the next tile's row max is folded 4 values per slot from slot NSM + MD,
        //    once its S MFMAs have completed.
        constexpr auto k_slot = [](int m) { return m - KA < -1 ? -1 : m - KA; };
        constexpr auto v_slot = [](int j) { return NSM + j - VA < -1 ? -1 : NSM + j - VA; };
        constexpr auto pair_slot = [](int j) {
            const int e = j * NSM / NPAIR - 1;
            const int deadline = NSM + (j / 4) * ND - 1;
            return e < deadline ? e : deadline;
        };
        constexpr auto reads_in_slot = [k_slot, v_slot](int p) {
            int n = 0;
            for (int m = 0; m < NSM; ++m) n += k_slot(m) == p;
            for (int j = 0; j < NPM; ++j) n += 2 * (v_slot(j) == p);
            return n;
        };
        // LDS reads (this wave's, in issue order) still allowed in flight when an
        // MFMA waits for its operand: those issued after it.
        constexpr auto k_pending = [k_slot, v_slot, reads_in_slot](int m) {
            const int p = k_slot(m);
            int n = 0;
            for (int m2 = m + 1; m2 < NSM; ++m2) n += k_slot(m2) == p;
            for (int j = 0; j < NPM; ++j) n += 2 * (v_slot(j) == p);
            for (int q = p + 1; q <= m - 1; ++q) n += reads_in_slot(q);
            return n;
        };
        constexpr auto v_pending = [v_slot, reads_in_slot](int j) {
            const int p = v_slot(j);
            int n = 0;
            for (int j2 = j + 1; j2 < NPM; ++j2) n += 2 * (v_slot(j2) == p);
            for (int q = p + 1; q <= NSM + j - 1; ++q) n += reads_in_slot(q);
            return n;
        };

        // One step: softmax and PV of tile kt (scores `cur`, V in stage PAR) with
        // S of tile kt+1 (into `nxt`, K in stage PAR ^ 1) interleaved; returns the
        // next tile's scaled row max. A tile hidden from the whole wave runs with
        // base = +inf, so every P is 0 (its scores must be finite).
        auto body = [&](auto par_tag, f32x16 (&cur)[NKT], f32x16 (&nxt)[NKT], bool hidden) {
            constexpr int PAR = decltype(par_tag)::value;
            const float base = hidden ? INFINITY : (m_run == -INFINITY) ? 0.0f : m_run;
            u32x4 kr[NSM];
            u32x2 vr[NPM][2];
            uint32_t pb[NPAIR];
            float mxa = -INFINITY, mxb = -INFINITY;
            auto issue_reads = [&](auto p_tag) {
                constexpr int p = decltype(p_tag)::value;
                static_for<NSM>([&](auto m_tag) {
                    if constexpr (k_slot(decltype(m_tag)::value) == p)
                        kr[m_tag] = k_read(std::integral_constant<int, PAR ^ 1>{}, m_tag);
                });
                static_for<NPM>([&](auto j_tag) {
                    if constexpr (v_slot(decltype(j_tag)::value) == p) v_read(par_tag, j_tag, vr[j_tag]);
                });
            };
            auto slot_valu = [&](auto p_tag) {
                constexpr int p = decltype(p_tag)::value;
                static_for<NPAIR>([&](auto j_tag) {
                    constexpr int j = decltype(j_tag)::value;
                    if constexpr (pair_slot(j) == p) {
                        constexpr int s = j / 4, i = j % 4, o8 = 8 * (s & 1);
                        const float e0 = exp2_fast(fmaf(cur[s >> 1][o8 + 2 * i], sl2e, -base));
                        const float e1 = exp2_fast(fmaf(cur[s >> 1][o8 + 2 * i + 1], sl2e, -base));
                        pb[j] = pack2<T>(e0, e1);
                        l_run = sum2<T>(pb[j], l_run);
                    }
                });
                if constexpr (p >= NSM + MD && 4 * (p - NSM - MD) < 16 * NKT) {
                    constexpr int r0 = 4 * (p - NSM - MD);
#pragma unroll
                    for (int r = r0; r < r0 + 4; r += 2) {
                        mxa = fmaxf(mxa, nxt[r / 16][r % 16]);
                        mxb = fmaxf(mxb, nxt[r / 16][r % 16 + 1]);
                    }
                }
            };

            issue_reads(std::integral_constant<int, -1>{});
            slot_valu(std::integral_constant<int, -1>{});
            static_for<NM>([&](auto m_tag) {
                constexpr int m = decltype(m_tag)::value;
                if constexpr (m < NSM) {
                    lds_wait4<k_pending(m)>(kr[m]);
                    nxt[m % NKT] = mfma16<T>(kr[m], qf[m / NKT], m < NKT ? f32x16{} : nxt[m % NKT]);
                } else {
                    constexpr int j = m - NSM, s = j / ND, t = j % ND;
                    lds_wait<v_pending(j)>(vr[j]);
                    const u32x4 a = {vr[j][0][0], vr[j][0][1], vr[j][1][0], vr[j][1][1]};
                    const u32x4 b = {pb[4 * s], pb[4 * s + 1], pb[4 * s + 2], pb[4 * s + 3]};
                    oacc[t] = mfma16<T>(a, b, oacc[t]);
                }
                issue_reads(m_tag);
                slot_valu(m_tag);
            });
            // The part of the max the slots did not cover.
            constexpr int done = NPM > MD ? 4 * (NPM - MD) : 0;
#pragma unroll
            for (int r = done < 16 * NKT ? done : 16 * NKT; r < 16 * NKT; r += 2) {
                mxa = fmaxf(mxa, nxt[r / 16][r % 16]);
                mxb = fmaxf(mxb, nxt[r / 16][r % 16 + 1]);
            }
            return half_max(fmaxf(mxa, mxb)) * sl2e;
        };

        // Step for tile kt at stage parity PAR = (kt - kt_begin) & 1: copies of
        // K(kt+2) and V(kt+1), then the body. The next tile's S is computed even
        // when it is hidden from this wave (or lies past the end: stale but finite
        // LDS data), so the common path has no branch around MFMA work; its max is
        // then discarded.
        int cls_cur = cls_of(kt_begin);
        float mt = -INFINITY;  // scaled row max of the current tile
        auto step = [&](auto par_tag, int kt, f32x16 (&cur)[NKT], f32x16 (&nxt)[NKT]) {
            constexpr int PAR = decltype(par_tag)::value;
            if (kt + 2 < kt_end) copy_k(kt + 2, PAR);
            if (kt + 1 < kt_end) copy_v(kt + 1, PAR ^ 1);
            const int cls_next = cls_of(kt + 1);
            float mt_next = -INFINITY;
            if (cls_cur != kEmpty || cls_next != kEmpty) {
                if (wave_any(mt > m_run + kRescaleLog2)) {
                    const float m_new = fmaxf(m_run, mt);
                    const float alpha = (m_run == -INFINITY) ? 0.0f : exp2_fast(m_run - m_new);
                    l_run *= alpha;
#pragma unroll
                    for (int t = 0; t < ND; ++t) oacc[t] *= alpha;
                    m_run = m_new;
                }
                mt_next = body(par_tag, cur, nxt, cls_cur == kEmpty);
            } else {
                // Both hidden: the next step may run this tile with P = 0, which
                // needs finite scores.
#pragma unroll
                for (int t = 0; t < NKT; ++t) nxt[t] = f32x16{};
            }
            if (cls_next == kEdge) {
                mask_tile(nxt, (kt + 1) * BN);
                mt_next = tile_max(nxt);
            }
            mt = cls_next == kEmpty ? -INFINITY : mt_next;
            cls_cur = cls_next;
            if (kt + 1 < kt_end) wait_copies();  // this wave's part of K(kt+2), V(kt+1)
            __syncthreads();                     // ... and everyone's; stages PAR free again
        };

        // Prologue: K and V of the first tile, K of the second, and S of the first.
        f32x16 sa[NKT], sb[NKT];
        __syncthreads();  // LDS zeroed before the first copy lands
        copy_k(kt_begin, 0);
        copy_v(kt_begin, 0);
        if (kt_begin + 1 < kt_end) copy_k(kt_begin + 1, 1);
        wait_copies();
        __syncthreads();
        if (cls_cur != kEmpty) {
            s_only(std::integral_constant<int, 0>{}, sa);
            if (cls_cur == kEdge) mask_tile(sa, kt_begin * BN);
            mt = tile_max(sa);
        } else {
#pragma unroll
            for (int t = 0; t < NKT; ++t) sa[t] = f32x16{};
        }
        __syncthreads();  // every wave has read K(kt_begin) before its stage is refilled
        // Unrolled by two, so the stage parity (and with it every LDS offset) is a
        // compile-time constant and the score buffers swap roles without copies.
        for (int kt = kt_begin;;) {
            step(std::integral_constant<int, 0>{}, kt, sa, sb);
            if (++kt == kt_end) break;
            step(std::integral_constant<int, 1>{}, kt, sb, sa);
            if (++kt == kt_end) break;
        }
        store_out(it0);
    } else {
        constexpr int NPV = BN / 16;  // PV k-steps per tile
        constexpr int NVR = 2 * ND;   // transposing V reads per PV k-step

        // Persistent walk: with fewer workgroups than work items (one per
        // resident slot, a multiple of 8), workgroup w takes in round r the
        // item of slot r C + (r even ? w / 8 : C - 1 - w / 8) on its own XCD
        // (item = 8 slot + w % 8, C = grid / 8). The item order (group by
        // group, each group's query tiles longest first) is walked forward,
        // then back, so a workgroup's long and short items alternate and the
        // totals balance; every item keeps the XCD the item order intends.
        // During an item's last tile the next item's first K/V tile and Q
        // rows are already on the way.
        const int n_slot = gridDim.x / 8, xcd = blockIdx.x % 8, slot0 = blockIdx.x / 8;
        const bool walk = TL::WALK && p.walk && gridDim.x % 8 == 0 && (int)gridDim.x < p.n_items;
        auto item_index = [&](int r) {
            return (r * n_slot + ((r & 1) ? n_slot - 1 - slot0 : slot0)) * 8 + xcd;
        };
        // This wave's Q rows of item `it` go global -> LDS (the wave reads them
        // back itself, after its own copies have landed). The resource starts
        // at the wave's first row (clamped to the sequence) and ends at its
        // last row in the sequence; rows past the end read row S - 1.
        uint8_t *const q_lds = lds + TL::LDS_BYTES + (TL::WALK ? wave * D * 64 : 0);
        auto copy_q = [&](const WaveItem &it) {
            const int r0 = min(it.wrow0, S - 1), r1 = min(it.wrow0 + 31, S - 1);
            const uint32_t row_bytes = (uint32_t)q_row_stride * 2;
            const uint8_t *base = static_cast<const uint8_t *>(p.q) +
                                  (((int64_t)it.b * S + r0) * q_row_stride + (int64_t)it.h * D) * 2;
            const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(base), 0, (int)((r1 - r0) * row_bytes + D * 2), kRsrcWord3);
            const uint32_t voff = (uint32_t)(min(it.row, S - 1) - r0) * row_bytes + 16 * g;
            if constexpr (TL::WALK) {
#pragma unroll
                for (int s = 0; s < D / 16; ++s) lds_copy16(rq, q_lds + s * 1024, voff + 32 * s);
            }
        };
        auto kbase = [&](const WaveItem &it) { return static_cast<const uint8_t *>(p.k) + it.kv_head0; };
        auto vbase = [&](const WaveItem &it) { return static_cast<const uint8_t *>(p.v) + it.kv_head0; };

        WaveItem cur = it0;
        int rnd = 0, kt = kt_begin, stage = 0;
        __syncthreads();  // LDS zeroed before the first copy lands
        copy_tile(Kbh, Vbh, kt, 0);
        land_tile(0);
        __syncthreads();

        for (;;) {
            const bool last = kt + 1 == cur.kt_end;
            const int next_idx = walk && last ? item_index(rnd + 1) : p.n_items;
            const bool more = next_idx < p.n_items;
            WaveItem nxt = cur;
            if (!last) {
                copy_tile(kbase(cur), vbase(cur), kt + 1, stage ^ 1);
            } else if (more) {
                nxt = wave_item<D, MASK, BN>(p, next_idx, wave, c32);
                copy_tile(kbase(nxt), vbase(nxt), nxt.kt_begin, stage ^ 1);
                copy_q(nxt);
            }
            const int wrow0 = cur.wrow0, row = cur.row;

            const int k0 = kt * BN;
            const int cls = classify<MASK>(wrow0, k0, k0 + BN - 1, S, W);
            if (cls != kEmpty) {
                // S^T = K Q^T: MFMA m takes k-step m / NKT of sub-tile m % NKT; its
                // K operand is read KA MFMAs ahead (explicit reads and counted
                // waits, so the schedule does not depend on the compiler's).
                constexpr int NSM = D / 16 * NKT;
                constexpr int KA = NSM < 4 ? NSM : 4;
                const uint32_t k_stage = lds_base + stage * TL::STAGE_BYTES;
                uint32_t kb[NKT][KP];
#pragma unroll
                for (int t = 0; t < NKT; ++t)
#pragma unroll
                    for (int q = 0; q < KP; ++q) kb[t][q] = k_stage + k_addr[t][q];
                auto k_read = [&](auto m_tag) {
                    constexpr int m = decltype(m_tag)::value, s = m / NKT, t = m % NKT;
                    return lds_read_b128<(s / KP) * 2 * KP * G * 16>(kb[t][s % KP]);
                };
                f32x16 sacc[NKT];
                u32x4 kr[NSM];
                // With a pre-scaled Q the accumulators start at -m (the
                // running max, or 0 before the first visible score).
                const float base0 = (m_run == -INFINITY) ? 0.0f : m_run;
                const f32x16 init = PRE ? f32x16{} - base0 : f32x16{};
                static_for<KA>([&](auto m_tag) { kr[m_tag] = k_read(m_tag); });
                static_for<NSM>([&](auto m_tag) {
                    constexpr int m = decltype(m_tag)::value;
                    lds_wait4<(m + KA <= NSM ? KA : NSM - m) - 1>(kr[m]);
                    sacc[m % NKT] = mfma16<T>(kr[m], qf[m / NKT], m < NKT ? init : sacc[m % NKT]);
                    if constexpr (m + KA < NSM) kr[m + KA] = k_read(std::integral_constant<int, m + KA>{});
                });

                // Edge tiles only: hidden scores become -inf, so exp2 gives them
                // exactly 0 below (the scale is never below 1e-30).
                // Element (t, r) holds key k0 + 4g + off, with the compile-time
                // offset off = 32t + 8(r/4) + r%4. The lane's visible offsets form
                // one range [lo, hi], so an element costs a compare and a select
                // (the window test is one unsigned compare against the span).
                if (cls == kEdge) {
                    int lo, hi;
                    visible_range<MASK>(row, k0 + 4 * g, S, W, BN, lo, hi);
                    const uint32_t span = (uint32_t)(hi - lo);
#pragma unroll
                    for (int t = 0; t < NKT; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = 32 * t + 8 * (r >> 2) + (r & 3);
                            const bool vis = MASK == kMaskWindow ? (uint32_t)(off - lo) <= span : off <= hi;
                            if (!vis) sacc[t][r] = -INFINITY;
                        }
                }

                // V^T operands. By k-step (D <= 64): the reads for PV k-steps
                // s .. s+V_AHEAD-1 are in flight while the exponentials of step s
                // are computed. By MFMA (D = 128 and 256): the two reads of PV
                // MFMA j (k-step j / ND, 32-dim sub-tile j % ND) are issued VJ
                // MFMAs ahead.
                const uint32_t v_region = lds_base + stage * TL::STAGE_BYTES + TL::TILE_BYTES;
                uint32_t v_stage[VT][VH];
#pragma unroll
                for (int tb = 0; tb < VT; ++tb)
#pragma unroll
                    for (int hb = 0; hb < VH; ++hb) v_stage[tb][hb] = v_region + v_addr[tb][hb];
                constexpr int NPM = NPV * ND, VJ = TL::V_PAIRS_AHEAD;
                u32x2 vr[NPM][2];  // the two reads of PV MFMA j
                auto issue_pair = [&](auto j_tag) {
                    constexpr int j = decltype(j_tag)::value;
                    if constexpr (j < NPM) {
                        constexpr int s = j / ND, t = j % ND;
                        constexpr int toff = (t - t % VT) * 64 * G;
                        constexpr int lo = (16 * s) / G * 1024 + toff;
                        constexpr int hi = (16 * s + 8 * (1 - 1 % VH)) / G * 1024 + toff;
                        vr[j][0] = lds_read_tr16<lo>(v_stage[t % VT][0]);
                        vr[j][1] = lds_read_tr16<hi>(v_stage[t % VT][1 % VH]);
                    }
                };
                auto issue_v = [&](auto s_tag) {
                    constexpr int s = decltype(s_tag)::value;
                    static_for<ND>([&](auto t_tag) { issue_pair(std::integral_constant<int, s * ND + t_tag>{}); });
                };
                if constexpr (VJ > 0)
                    static_for<VJ>(issue_pair);
                else
                    static_for<V_AHEAD>(issue_v);

                // Running max; raised (and O, l rescaled) only when it grows by
                // more than 2^kRescaleLog2.
                float mx = -INFINITY;
#pragma unroll
                for (int t = 0; t < NKT; ++t)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
                float base = 0.0f;
                if constexpr (PRE) {
                    // Scores are already exponents relative to base0: raise the
                    // max when a row's first scores arrive or when this tile's
                    // max exceeds it by more than 2^kRescaleLog2, and move the
                    // tile's exponents to the new max.
                    const float mt = half_max(mx);
                    if (wave_any(m_run == -INFINITY ? mt != -INFINITY : mt > kRescaleLog2)) {
                        const float delta = mt == -INFINITY ? 0.0f : (m_run == -INFINITY ? mt : fmaxf(mt, 0.0f));
                        const float alpha = (m_run == -INFINITY) ? 0.0f : exp2_fast(-delta);
                        l_run *= alpha;
#pragma unroll
                        for (int t = 0; t < ND; ++t) oacc[t] *= alpha;
                        if (mt != -INFINITY) m_run = base0 + delta;
#pragma unroll
                        for (int t = 0; t < NKT; ++t) sacc[t] -= delta;
                    }
                } else {
                    const float mt = half_max(mx) * sl2e;
                    if (wave_any(mt > m_run + kRescaleLog2)) {
                        const float m_new = fmaxf(m_run, mt);
                        const float alpha = (m_run == -INFINITY) ? 0.0f : exp2_fast(m_run - m_new);
                        l_run *= alpha;
#pragma unroll
                        for (int t = 0; t < ND; ++t) oacc[t] *= alpha;
                        m_run = m_new;
                    }
                    base = (m_run == -INFINITY) ? 0.0f : m_run;
                }

                // P = exp2(s * scale log2e - m), rounded to T; l += sum of the
                // rounded values; O^T += V^T P^T.
                static_for<NPV>([&](auto s_tag) {
                    constexpr int s = decltype(s_tag)::value;
                    constexpr int o8 = 8 * (s & 1);
                    u32x4 pb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x0 = sacc[s >> 1][o8 + 2 * i], x1 = sacc[s >> 1][o8 + 2 * i + 1];
                        const float e0 = exp2_fast(PRE ? x0 : fmaf(x0, sl2e, -base));
                        const float e1 = exp2_fast(PRE ? x1 : fmaf(x1, sl2e, -base));
                        pb[i] = pack2<T>(e0, e1);
                        l_run = sum2<T>(pb[i], l_run);
                    }
                    if constexpr (VJ > 0) {
                        static_for<ND>([&](auto t_tag) {
                            constexpr int t = decltype(t_tag)::value, j = s * ND + t;
                            // Pairs j+1 .. j+VJ-1 (those that exist) may pend.
                            constexpr int later = (NPM - 1 - j < VJ - 1) ? NPM - 1 - j : VJ - 1;
                            lds_wait<2 * later>(vr[j]);
                            const u32x4 a = {vr[j][0][0], vr[j][0][1], vr[j][1][0], vr[j][1][1]};
                            oacc[t] = mfma16<T>(a, pb, oacc[t]);
                            issue_pair(std::integral_constant<int, j + VJ>{});
                        });
                    } else {
                        // Step s+1's reads may pend.
                        constexpr int later = (V_AHEAD > 1 && s + 1 < NPV) ? NVR : 0;
                        lds_wait<later>(vr[s * ND]);
#pragma unroll
                        for (int t = 1; t < ND; ++t) {
                            lds_tie(vr[s * ND + t][0]);
                            lds_tie(vr[s * ND + t][1]);
                        }
#pragma unroll
                        for (int t = 0; t < ND; ++t) {
                            const u32x4 a = {vr[s * ND + t][0][0], vr[s * ND + t][0][1], vr[s * ND + t][1][0],
                                             vr[s * ND + t][1][1]};
                            oacc[t] = mfma16<T>(a, pb, oacc[t]);
                        }
                        issue_v(std::integral_constant<int, s + V_AHEAD>{});
                    }
                });
            }

            if (!last || more) land_tile(stage ^ 1);  // this wave's part of the next tile (and its Q rows)
            if (last) {
                store_out(cur);
                if (!more) break;
                m_run = -INFINITY;
                l_run = 0.0f;
#pragma unroll
                for (int t = 0; t < ND; ++t) oacc[t] = f32x16{};
                if constexpr (TL::WALK) {
#pragma unroll
                    for (int s = 0; s < D / 16; ++s) {
                        qf[s] = *reinterpret_cast<const u32x4 *>(q_lds + s * 1024 + 16 * lane) ^ p.q_sign;
                        if constexpr (PRE) qf[s] = scale_frag<T>(qf[s], p.scale_log2);
                    }
                }
                cur = nxt;
                kt = cur.kt_begin;
                ++rnd;
            } else {
                ++kt;
            }
            stage ^= 1;
            __syncthreads();  // ... and everyone's; the current stage is free again
        }
    }

}

}  // namespace fa355
