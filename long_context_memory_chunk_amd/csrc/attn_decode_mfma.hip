// Stage 3 for decode and short queries (bf16, d = 128, G = Hq/Hkv <= 8), with
// the scores on the matrix cores.
//
// Source: news.neo-ai.one MSA article, 全体設計 › アーキテクチャ (Fig. 2) and
// 推論パイプライン (Fig. 3), third stage: a generated token attends over the
// selected K̄/V̄ rows and its local K/V, global RoPE shifting its start by k.
// Key space, positions and mask are those of attn.hip.
//
// A workgroup (4 waves) owns one (query token, KV head g) and a run of NC
// 128-key chunks; wave w takes keys 32w .. 32w+31 of every chunk and the four
// waves' online softmaxes meet once at the end in one partial (m, l, o) per
// workgroup, which attn_combine merges with the others.  Per 32-key block a
// wave
//   * loads its K rows with each lane holding dimensions 4c .. 4c+3 and their
//     RoPE partners 64 + 4c .. (c = lane % 16, four rows per instruction, 128
//     contiguous bytes per row), rotates a local key in the lane at position
//     q_offset + j (cos/sin seeded from the table and advanced by a fixed
//     4-position rotation from row to row), and stores the rows to a
//     per-wave LDS tile (16-byte units XOR-swizzled by row);
//   * forms S = Q . K^T with eight v_mfma_f32_32x32x16_bf16: the A operand
//     holds the G rotated query heads (scale and log2(e) folded in) in its
//     first G rows and zeros elsewhere, the B operand reads lane l's key
//     l % 32, dimensions 16 s + 8 (l / 32) .. +7 of step s, from the tile.
//     The dot products, and the reductions across lanes they would need,
//     leave the vector units; head h's 32 scores land in register h % 4 of
//     lanes 32 (h / 4) .. +31, one key per lane;
//   * runs the online softmax per head in the log2 domain: the running max is
//     raised only when a ballot finds a score past m + 8 (the block max is
//     reduced only then), and each lane sums its own probabilities;
//   * passes P through LDS as bf16 pairs (keys 2p, 2p + 1) and forms
//     O += P . V on the vector units with v_dot2 over those pairs: a lane
//     holds value rows 2 slot + 8 m and 2 slot + 8 m + 1 (m = 0 .. 3,
//     slot = lane / 16), dimensions 8 (lane % 16) .. +7, so each 16-byte load
//     instruction reads four whole rows, and a byte permute puts the two
//     rows' values of one dimension side by side.
// A block wholly in the memory rows, or wholly in the local rows before the
// end, is addressed from a wave-uniform base plus 32-bit lane offsets.  The
// next block's K rows are loaded once this block's tile is stored, and its V
// rows once this block's P . V is done.
#include "common.hpp"
#include "attn_mfma.hpp"
#include "gather_body.hpp"

namespace msa {

namespace {

typedef __bf16 bf16x8_d __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_d __attribute__((ext_vector_type(2)));
typedef float f32x16_d __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int DH = 128;
static_assert(kDecodeChunk == 128, "a chunk is 4 waves x 32 keys");
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;
constexpr float kLazyD = 8.f;

__device__ __forceinline__ bf16x8_d as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8_d, w); }
__device__ __forceinline__ bf16x2_d as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_d, w); }

// Eight elements of one lane's RoPE pair runs (x1 = dims i.., x2 = dims
// i + 64..) rotated, (x1 c - x2 s, x2 c + x1 s), scaled and packed as two
// 16-byte matrix-core operands.
__device__ __forceinline__ void rotate_pack(u32x4 x1, u32x4 x2, const float2* __restrict__ cs, float sc,
                                            u32x4& y1p, u32x4& y2p) {
    float y1[8], y2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = (e & 1) ? bf16_hi(x1[e / 2]) : bf16_lo(x1[e / 2]);
        const float b = (e & 1) ? bf16_hi(x2[e / 2]) : bf16_lo(x2[e / 2]);
        const float2 r = cs[e];
        y1[e] = (a * r.x - b * r.y) * sc;
        y2[e] = (b * r.x + a * r.y) * sc;
    }
    y1p = u32x4{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]), pack_bf16x2(y1[4], y1[5]),
                pack_bf16x2(y1[6], y1[7])};
    y2p = u32x4{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]), pack_bf16x2(y2[4], y2[5]),
                pack_bf16x2(y2[6], y2[7])};
}

// The arguments of one launch.  Partials of row r and partition p of this
// launch go to index r * P_total + p_base + p of part_o / part_ml, so two
// launches over disjoint key ranges of the same rows fill one partial set.
struct DecodeArgs {
    const uint16_t* Q;
    int Tq, Hq, hkv;
    const uint16_t* KVmem;
    const int64_t* mem_off;
    int64_t cap, max_rows;
    const uint16_t* Kl;
    const uint16_t* Vl;
    int L, q_offset;
    float qscale;
    const float2* rope_cs;
    int max_pos;
    int NC, p_base, P_total;
    int use_mem, use_local;   // 1/1 all keys, 0/1 local keys only, 1/0 memory rows only (launch
                              // arguments: every range runs the one compiled body)
    float* part_o;
    float2* part_ml;
};

// Key ranges: every key of the row, only its local keys (memory rows taken as
// absent: neither KVmem nor mem_off is read), or only its memory rows.  The
// query keeps its position in every case.
enum DecodeKeys : int { kKeysAll = 0, kKeysLocal = 1, kKeysMem = 2 };

// One workgroup: partition p (chunks p * NC ..) of (query token bt, KV head g);
// P is the partials' row stride and p_base + p this partial's index.  (The
// pointers are parameters so that their no-alias promise survives inlining.)
template <int G, bool kRanged>
__device__ __forceinline__ void decode_wg(
    const uint16_t* __restrict__ Q, int Tq, int Hq, int hkv, const uint16_t* __restrict__ KVmem,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows, const uint16_t* __restrict__ Kl,
    const uint16_t* __restrict__ Vl, int L, int q_offset, float qscale, const float2* __restrict__ rope_cs,
    int max_pos, int NC, int p_base, int P, int use_mem, int use_local, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int p, int g, int64_t bt) {
    const int pp = p_base + p;
    constexpr int GH = G < 4 ? G : 4;             // heads per 32-lane half of the score layout
    __shared__ u32x4 s_k[4][32 * 16];             // each wave's 32 (rotated) key rows, 16-byte units swizzled
    __shared__ uint32_t s_pp[4][16][G];           // P of each wave's block: pair p = keys 2p, 2p + 1
    __shared__ float red[4][G][DH];
    __shared__ float s_m[4][G], s_l[4][G];

    const int tid = threadIdx.x, lane = tid % kWave, half = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int slot = lane / 16, c = lane % 16;    // row layouts: 4 rows per instruction
    const int col = lane % 32;                    // score layout: key (B operand column), head (A operand row)
    const int64_t b = bt / Tq;
    const int i = int(bt % Tq);

    int64_t r0 = 0, M = 0;
    // (the all-keys kernel is compiled without the range; a local-keys range
    // does not read mem_off, which a copy in the same launch may be writing)
    if (!kRanged || use_mem) mem_range(mem_off, b, cap, max_rows, r0, M);
    const int64_t total = M + (kRanged ? use_local : 1) * (int64_t(L - Tq) + i + 1);
    const int64_t row_elems = int64_t(hkv) * DH;
    const int64_t hrow = bt * Hq + int64_t(g) * G;   // first query head row of this group
    const int64_t n_chunks = (total + kDecodeChunk - 1) / kDecodeChunk;
    const int64_t cb = int64_t(p) * NC;
    const int64_t ce = (cb + NC < n_chunks) ? cb + NC : n_chunks;

    if (cb >= ce) {                               // no keys here: an empty partial
        for (int idx = tid; idx < G * DH; idx += 256) part_o[((hrow + idx / DH) * P + pp) * DH + idx % DH] = 0.f;
        if (tid < G) part_ml[(hrow + tid) * P + pp] = make_float2(-INFINITY, 0.f);
        return;
    }

    // ---- A operands: row col < G is query head hrow + col, rotated at its
    // position and scaled; the other rows are zero
    bf16x8_d qa[8];
    {
        const uint16_t* qrow = Q + (hrow + (col < G ? col : 0)) * DH;
        int pos = q_offset + (L - Tq) + i;
        pos = pos < max_pos ? pos : max_pos - 1;
        const float2* cs = rope_cs + int64_t(pos) * (DH / 2);
        const float sc = col < G ? qscale : 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c0 = 16 * s + 8 * half;
            u32x4 y1, y2;
            rotate_pack(*reinterpret_cast<const u32x4*>(qrow + c0), *reinterpret_cast<const u32x4*>(qrow + c0 + DH / 2),
                        cs + c0, sc, y1, y2);
            qa[s] = as_bf16x8(y1);
            qa[s + 4] = as_bf16x8(y2);
        }
    }

    // Row addresses.  A block that lies wholly in the memory rows, or wholly in
    // the local rows before the end, is addressed from a wave-uniform base plus
    // a 32-bit lane offset; a block across the boundary or the end goes row by
    // row, rows past the end clamped to the last key (and masked).
    const char* kv_g = reinterpret_cast<const char*>(KVmem + int64_t(g) * DH);
    const char* kl_g = reinterpret_cast<const char*>(Kl + int64_t(g) * DH);
    const char* vl_g = reinterpret_cast<const char*>(Vl + int64_t(g) * DH);
    const int64_t mem_stride = 2 * row_elems * 2, loc_stride = row_elems * 2;   // bytes per row
    const int64_t loc_row0 = b * L - M;           // local row of key kk: loc_row0 + kk
    auto row_ptr = [&](int64_t key, bool value) {
        key = key < total ? key : total - 1;
        return (key >= M) ? (value ? vl_g : kl_g) + (loc_row0 + key) * loc_stride
                          : kv_g + (r0 + key) * mem_stride + (value ? row_elems * 2 : 0);
    };
    // K rows slot + 4 it (it = 0 .. 7) of a block: lane c holds dimensions
    // 4c .. 4c+3 and their RoPE partners 64 + 4c .. 64 + 4c + 3, so each load
    // instruction reads 128 contiguous bytes of four rows and the rotation stays
    // in the lane; the cos/sin of the lane's first local row ("seed") advance
    // by the fixed rotation of 4 positions from row to row.
    u32x2 kw[8][2];
    float2 seed[4], step[4];
    u32x4 vw[8];
    {
        const float2* st = rope_cs + int64_t(4 < max_pos ? 4 : max_pos - 1) * (DH / 2) + 4 * c;
#pragma unroll
        for (int j = 0; j < 4; ++j) step[j] = st[j];
    }
    auto first_local = [&](int64_t k0) {          // the lane's first row it with key >= M
        const int64_t kb = k0 + slot;
        return (M > kb) ? (M - kb + 3) / 4 : int64_t(0);
    };
    auto load_k = [&](int64_t k0) {
        // the RoPE seed first: an address it needs may have to come back from
        // scratch, and that wait then does not cover this block's K loads
        if (k0 + 31 >= M) {                        // the block holds local keys
            int64_t pos = int64_t(q_offset) + k0 + slot + 4 * first_local(k0) - M;
            pos = pos < 0 ? 0 : (pos < max_pos ? pos : max_pos - 1);
            const float2* cs = rope_cs + pos * (DH / 2) + 4 * c;
#pragma unroll
            for (int j = 0; j < 4; ++j) seed[j] = cs[j];
        }
        if (k0 + 31 < M || (k0 >= M && k0 + 31 < total)) {
            const bool mem = k0 + 31 < M;
            const int64_t stride = mem ? mem_stride : loc_stride;
            const char* base = mem ? kv_g + (r0 + k0) * mem_stride : kl_g + (loc_row0 + k0) * loc_stride;
            const uint32_t vo = uint32_t(slot) * uint32_t(stride) + 8u * c;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const char* rb = base + 4 * it * stride + vo;
                kw[it][0] = *reinterpret_cast<const u32x2*>(rb);
                kw[it][1] = *reinterpret_cast<const u32x2*>(rb + DH);
            }
        } else {
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const char* rb = row_ptr(k0 + slot + 4 * it, false) + 8 * c;
                kw[it][0] = *reinterpret_cast<const u32x2*>(rb);
                kw[it][1] = *reinterpret_cast<const u32x2*>(rb + DH);
            }
        }
    };
    // V rows 2 slot + 8 m + q (it = 2m + q): lane c holds dimensions 8c .. 8c+7
    auto load_v = [&](int64_t k0) {
        if (k0 + 31 < M || (k0 >= M && k0 + 31 < total)) {
            const bool mem = k0 + 31 < M;
            const int64_t stride = mem ? mem_stride : loc_stride;
            const char* base = mem ? kv_g + (r0 + k0) * mem_stride + row_elems * 2 : vl_g + (loc_row0 + k0) * loc_stride;
            const uint32_t vo = uint32_t(2 * slot) * uint32_t(stride) + 16u * c;
#pragma unroll
            for (int it = 0; it < 8; ++it)
                vw[it] = *reinterpret_cast<const u32x4*>(base + (8 * (it / 2) + (it % 2)) * stride + vo);
        } else {
#pragma unroll
            for (int it = 0; it < 8; ++it)
                vw[it] = *reinterpret_cast<const u32x4*>(row_ptr(k0 + 2 * slot + 8 * (it / 2) + (it % 2), true) + 16 * c);
        }
    };
    char* tile_b = reinterpret_cast<char*>(s_k[wave]);
    const u32x4* tile = s_k[wave];

    float m_h[G];                                 // running max per head (the same in every lane)
    float l_lane[GH];                             // this lane's probability sums (its key of every block)
    float o[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m_h[hh] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < GH; ++j) l_lane[j] = 0.f;

    int64_t k0 = cb * kDecodeChunk + wave * 32;       // this wave's first key of the current chunk
    if (k0 < total) {
        load_k(k0);
        load_v(k0);
    }
    for (int64_t cc = cb; cc < ce; ++cc) {
        if (k0 >= total) break;                   // wave-uniform
        const int64_t kn = k0 + kDecodeChunk;
        const bool more = (cc + 1 < ce) && (kn < total);

        // ---- rotate the block's local rows, store the rows to the wave's tile
        // (16-byte unit u of row r at u ^ (r & 15)), then load the next block's K
        if (k0 + 31 >= M) {
            const int64_t fl = k0 >= M ? 0 : first_local(k0);
            float2 rot[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) rot[j] = seed[j];
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                if (it >= fl) {
                    if (it > fl) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float2 r = rot[j];
                            rot[j] = make_float2(r.x * step[j].x - r.y * step[j].y, r.y * step[j].x + r.x * step[j].y);
                        }
                    }
                    float y1[4], y2[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float a = (j & 1) ? bf16_hi(kw[it][0][j / 2]) : bf16_lo(kw[it][0][j / 2]);
                        const float bb = (j & 1) ? bf16_hi(kw[it][1][j / 2]) : bf16_lo(kw[it][1][j / 2]);
                        y1[j] = a * rot[j].x - bb * rot[j].y;
                        y2[j] = bb * rot[j].x + a * rot[j].y;
                    }
                    kw[it][0] = u32x2{pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3])};
                    kw[it][1] = u32x2{pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3])};
                }
            }
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = slot + 4 * it;
            const int u0 = (c >> 1) ^ (r & 15), u1 = (8 + (c >> 1)) ^ (r & 15);
            *reinterpret_cast<u32x2*>(tile_b + r * 256 + u0 * 16 + (c & 1) * 8) = kw[it][0];
            *reinterpret_cast<u32x2*>(tile_b + r * 256 + u1 * 16 + (c & 1) * 8) = kw[it][1];
        }
        if (more) load_k(kn);
        // Written and read by this wave only: its LDS accesses complete in order.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- S = Q . K^T (two accumulation chains where registers allow); the
        // B operand of step s is unit 2s + half of row col.  Register h % 4 of
        // lane 32 (h / 4) + j holds the score of head h and key j.
        constexpr bool kTwoChains = G < 4;
        f32x16_d s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
        for (int s = 0; s < 8; s += 2) {
            const bf16x8_d b0 = as_bf16x8(tile[col * 16 + ((2 * s + half) ^ (col & 15))]);
            const bf16x8_d b1 = as_bf16x8(tile[col * 16 + ((2 * s + 2 + half) ^ (col & 15))]);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], b0, s0, 0, 0, 0);
            if (kTwoChains)
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s + 1], b1, s1, 0, 0, 0);
            else
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s + 1], b1, s0, 0, 0, 0);
        }

        // ---- online softmax per head over the block's 32 keys (log2 domain).
        // The running max m of a head is raised only when some score passes
        // m + 8 (a ballot; the max itself is reduced only then); each lane sums
        // its own probabilities, and the lanes' sums are added once at the end.
        float sv[GH];
#pragma unroll
        for (int j = 0; j < GH; ++j) sv[j] = kTwoChains ? s0[j] + s1[j] : s0[j];
        if (k0 + 31 >= total) {                    // the last block: mask keys past the end
            const int nvalid = int(total - k0);
#pragma unroll
            for (int j = 0; j < GH; ++j) sv[j] = col < nvalid ? sv[j] : -INFINITY;
        }
        float corr[G];
        bool any_raise = false;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const int j = hh % 4, hl = hh / 4;     // register, lane half
            const uint64_t over = __builtin_amdgcn_ballot_w64(sv[j] > m_h[hh] + kLazyD) &
                                  (hl ? 0xFFFFFFFF00000000ull : 0x00000000FFFFFFFFull);
            corr[hh] = 1.f;
            if (over) {
                const float mx16 = group_max<16>(sv[j]);
                const float mb = fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx16), 32 * hl)),
                                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx16), 32 * hl + 16)));
                corr[hh] = m_h[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_h[hh] - mb);
                m_h[hh] = mb;
                any_raise = true;
            }
        }
#pragma unroll
        for (int j = 0; j < GH; ++j) {
            const bool up = G > 4 && half;         // lanes 32 .. 63 hold heads 4 .. 7
            const float mj = up ? m_h[(4 + j) % G] : m_h[j];
            const float cj = up ? corr[(4 + j) % G] : corr[j];
            sv[j] = __builtin_amdgcn_exp2f(sv[j] - mj);   // masked: exp2(-inf) = 0
            l_lane[j] = l_lane[j] * cj + sv[j];
        }
        // P as bf16 pairs of keys (2p, 2p + 1): the even lane packs its odd neighbour's value
        {
            uint32_t pk[GH];
#pragma unroll
            for (int j = 0; j < GH; ++j) pk[j] = pack_bf16x2(sv[j], dpp<kQuadXor1>(sv[j]));
            if ((col & 1) == 0 && (G > 4 || half == 0)) {
                uint32_t* dst = &s_pp[wave][col / 2][GH * half];
#pragma unroll
                for (int j = 0; j < GH; ++j) dst[j] = pk[j];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- O = O * corr + P . V
        if (any_raise) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[hh][e] *= corr[hh];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            uint32_t pp[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) pp[hh] = s_pp[wave][slot + 4 * m][hh];
            const u32x4 va = vw[2 * m], vb = vw[2 * m + 1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);   // (a[2w], b[2w])
                const uint32_t hi = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);   // (a[2w+1], b[2w+1])
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    o[hh][2 * w] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(lo), as_bf16x2(pp[hh]), o[hh][2 * w], false);
                    o[hh][2 * w + 1] =
                        __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(hi), as_bf16x2(pp[hh]), o[hh][2 * w + 1], false);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();          // this block's tile and P read before the next block writes them
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (more) load_v(kn);
        k0 = kn;
    }

    // ---- merge the four key slots of each wave, then the waves
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[hh][e];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            o[hh][e] = v;
        }
    if (slot == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][hh][c * 8 + e] = o[hh][e];
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        const int j = hh % 4, hl = hh / 4;
        const float s16 = group_sum<16>(l_lane[j]);
        const float lw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 32 * hl)) +
                         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s16), 32 * hl + 16));
        if (lane == 0) {
            s_m[wave][hh] = m_h[hh];
            s_l[wave][hh] = lw;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * DH; idx += 256) {
        const int hh = idx / DH, dd = idx % DH;
        const float mw = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = (s_m[w][hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][hh] - mw);
            acc += f * red[w][hh][dd];
        }
        part_o[((hrow + hh) * P + pp) * DH + dd] = acc;
    }
    if (tid < G) {
        const float mw = fmaxf(fmaxf(s_m[0][tid], s_m[1][tid]), fmaxf(s_m[2][tid], s_m[3][tid]));
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            lsum += (s_m[w][tid] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][tid] - mw) * s_l[w][tid];
        // the combine takes m in natural-log units
        part_ml[(hrow + tid) * P + pp] = make_float2(mw == -INFINITY ? -INFINITY : mw * kLn2D, lsum);
    }
}

template <int G>
__device__ __forceinline__ void decode_ranged(const DecodeArgs& da, int p, int g, int64_t bt) {
    decode_wg<G, true>(da.Q, da.Tq, da.Hq, da.hkv, da.KVmem, da.mem_off, da.cap, da.max_rows, da.Kl, da.Vl, da.L,
                       da.q_offset, da.qscale, da.rope_cs, da.max_pos, da.NC, da.p_base, da.P_total, da.use_mem,
                       da.use_local, da.part_o, da.part_ml, p, g, bt);
}

// Every key of each row (the arguments one by one, as the launch passes them).
template <int G>
__global__ __launch_bounds__(256, G < 8 ? 2 : 1) void attn_decode_mfma_kernel(
    const uint16_t* __restrict__ Q, int Tq, int Hq, int hkv, const uint16_t* __restrict__ KVmem,
    const int64_t* __restrict__ mem_off, int64_t cap, int64_t max_rows, const uint16_t* __restrict__ Kl,
    const uint16_t* __restrict__ Vl, int L, int q_offset, float qscale, const float2* __restrict__ rope_cs,
    int max_pos, int P, int NC, float* __restrict__ part_o, float2* __restrict__ part_ml) {
    decode_wg<G, false>(Q, Tq, Hq, hkv, KVmem, mem_off, cap, max_rows, Kl, Vl, L, q_offset, qscale, rope_cs, max_pos,
                        NC, 0, P, 1, 1, part_o, part_ml, int(blockIdx.x), int(blockIdx.y), int64_t(blockIdx.z));
}

// A key range of each row (memory rows only), partials at an offset.
template <int G>
__global__ __launch_bounds__(256, G < 8 ? 2 : 1) void attn_decode_range_kernel(DecodeArgs da) {
    decode_ranged<G>(da, int(blockIdx.x), int(blockIdx.y), int64_t(blockIdx.z));
}

// The eight bf16 values of a 16-byte unit (the dwords unpacked by name).
__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
    const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    f[0] = bf16_lo(w0); f[1] = bf16_hi(w0); f[2] = bf16_lo(w1); f[3] = bf16_hi(w1);
    f[4] = bf16_lo(w2); f[5] = bf16_hi(w2); f[6] = bf16_lo(w3); f[7] = bf16_hi(w3);
}

// One-query copy of destination rows wg * R .. wg * R + R - 1 that also forms
// the attention partial of those rows for every query head of a one-token
// query (index pp of its row's partials), so that the memory rows need no
// launch of their own after the copy.  A row is [K̄ ; V̄] of hkv heads, 32 hkv
// <= 256 units of 16 bytes: thread t copies unit t of every row and keeps it.
// Thread 16 g + c (t < 16 hkv) holds dimensions 8c .. 8c+7 of K̄ head g: it
// rotates the G query heads of group g at those dimensions (their RoPE
// partners 8 (c ^ 8) .. come from the same query row), forms its share of
// each row's score and sums the 16 shares of the group (fp32 throughout),
// and the group's lane 0 hands the probabilities to the V̄ threads through
// LDS; thread 16 hkv + 16 g + c then accumulates dimensions 8c .. 8c+7 of
// the G heads' outputs.  A workgroup past the gathered rows writes nothing:
// the combine reads the partials of the first ceil(mem_off[1] / R) only.
template <int G, int R>
__device__ __forceinline__ void gather_one_attn_wg(const GatherCopyArgs& gc, const DecodeArgs& da, int wg, int pp) {
    __shared__ float s_p[8][G][R];
    int64_t sr[R];
    gather_one_plan<R>(gc.ids, gc.K, gc.off, gc.n_docs, gc.n_rows_host, gc.cap, gc.mem_off, wg, sr);
    // past the gathered rows (the same answer in every wave): nothing to copy,
    // and the combine reads no partial of this workgroup
    if (sr[0] < 0) return;
    const int t = threadIdx.x;
    const int64_t rv = gc.row_vecs;
    const bool on = t < rv;
    const int64_t r0 = int64_t(wg) * R;
    u32x4 x[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        x[j] = u32x4{0u, 0u, 0u, 0u};
        if (on && sr[j] >= 0) x[j] = gc.host[sr[j] * rv + t];
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (on && sr[j] >= 0) gc.dst[(r0 + j) * rv + t] = x[j];

    const int P = da.P_total, kv_units = 16 * da.hkv, c = t % 16;
    if (t < kv_units) {
        const int g = t / 16;
        int pos = da.q_offset + da.L - 1;          // the token's global position (Tq = 1)
        pos = pos < da.max_pos ? pos : da.max_pos - 1;
        const float2* cs = da.rope_cs + int64_t(pos) * (DH / 2) + 8 * (c % 8);
        float s[R][G];
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int hh = 0; hh < G; ++hh) s[j][hh] = 0.f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            const uint16_t* qrow = da.Q + int64_t(g * G + hh) * DH;
            float a[8], b[8], q[8];
            unpack8(*reinterpret_cast<const u32x4*>(qrow + 8 * c), a);
            unpack8(*reinterpret_cast<const u32x4*>(qrow + 8 * (c ^ 8)), b);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float2 r = cs[e];
                q[e] = (c < 8 ? a[e] * r.x - b[e] * r.y : a[e] * r.x + b[e] * r.y) * da.qscale;
            }
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float k[8];
                unpack8(x[j], k);
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += q[e] * k[e];
                s[j][hh] = d;
            }
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float m = -INFINITY;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                s[j][hh] = group_sum<16>(s[j][hh]);
                if (sr[j] < 0) s[j][hh] = -INFINITY;
                m = fmaxf(m, s[j][hh]);
            }
            float l = 0.f, p[R];
#pragma unroll
            for (int j = 0; j < R; ++j) {
                p[j] = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s[j][hh] - m);
                l += p[j];
            }
            if (c == 0) {
#pragma unroll
                for (int j = 0; j < R; ++j) s_p[g][hh][j] = p[j];
                // the combine takes m in natural-log units
                da.part_ml[int64_t(g * G + hh) * P + pp] = make_float2(m == -INFINITY ? -INFINITY : m * kLn2D, l);
            }
        }
    }
    __syncthreads();
    if (t >= kv_units && on) {
        const int g = (t - kv_units) / 16;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float pj = s_p[g][hh][j];
                float v[8];
                unpack8(x[j], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] += pj * v[e];
            }
            float4* op = reinterpret_cast<float4*>(da.part_o + (int64_t(g * G + hh) * P + pp) * DH + 8 * c);
            op[0] = make_float4(o[0], o[1], o[2], o[3]);
            op[1] = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
}

// The device gather and the attention over the local keys in one launch: the
// copy waits on PCIe and leaves most CUs idle, and the local keys (most of a
// decode row's keys) need none of the gathered rows, so their partials are
// formed meanwhile.  Workgroups [copy_first, copy_first + n_copy) copy, the
// others are the local-key attention grid (P x hkv x B*Tq, partition
// fastest).  The bounded copy goes first, since it is the longer; the
// one-query copy (one workgroup per kOneRows rows) after the attention, so
// that a large capacity cannot hold every slot before the attention starts.
// With attn_rows (a one-token query: 4 or 8; 0 for the copy alone) the
// one-query copy takes attn_rows rows per workgroup and also forms their
// partials (indices P + wg), so the launch covers every key of the row.
template <int G, bool kOne>
__global__ __launch_bounds__(256, G < 8 ? 2 : 1) void gather_local_attn_kernel(GatherCopyArgs gc, DecodeArgs da,
                                                                              int P, int copy_first, int n_copy,
                                                                              int attn_rows) {
    const int bx = int(blockIdx.x);
    if (bx >= copy_first && bx < copy_first + n_copy) {
        const int wg = bx - copy_first;
        if (kOne && attn_rows == kOneAttnRowsFew)
            gather_one_attn_wg<G, kOneAttnRowsFew>(gc, da, wg, P + wg);
        else if (kOne && attn_rows == kOneAttnRowsMany)
            gather_one_attn_wg<G, kOneAttnRowsMany>(gc, da, wg, P + wg);
        else if (kOne)
            gather_one_wg(gc.host, gc.row_vecs, gc.ids, gc.K, gc.off, gc.n_docs, gc.n_rows_host, gc.cap, gc.mem_off,
                          gc.dst, wg);
        else
            gather_copy_wg(gc.host, gc.row_vecs, gc.src_of_row, gc.mem_off, gc.B, gc.dst, wg, n_copy);
        return;
    }
    // 32-bit, wave-uniform index arithmetic (the grid has fewer than 2^31 workgroups)
    const uint32_t w = uint32_t(__builtin_amdgcn_readfirstlane(bx < copy_first ? bx : bx - n_copy));
    // (the divisions run on the vector units: readfirstlane puts their results
    // back in scalar registers, so the addresses built from them stay scalar)
    const uint32_t wp = uint32_t(__builtin_amdgcn_readfirstlane(int(w / uint32_t(P))));
    const int p = __builtin_amdgcn_readfirstlane(int(w - wp * uint32_t(P)));
    const int g = __builtin_amdgcn_readfirstlane(int(wp % uint32_t(da.hkv)));
    const int bt = __builtin_amdgcn_readfirstlane(int(wp / uint32_t(da.hkv)));
    decode_ranged<G>(da, p, g, int64_t(bt));
}

DecodeArgs decode_args(const AttnArgs& a, int keys, float* part_o, float2* part_ml, int nc, int p_base,
                       int P_total) {
    return DecodeArgs{static_cast<const uint16_t*>(a.Q), a.Tq, a.Hq, a.Hkv, static_cast<const uint16_t*>(a.KVmem),
                      a.mem_off, a.mem_rows_cap, a.max_rows, static_cast<const uint16_t*>(a.K_local),
                      static_cast<const uint16_t*>(a.V_local), a.L, a.q_offset, a.scale * kLog2eD, a.rope_cs,
                      a.max_pos, nc, p_base, P_total, keys != kKeysLocal, keys != kKeysMem, part_o, part_ml};
}

hipError_t launch_range(const AttnArgs& a, const DecodeArgs& da, int P, hipStream_t st) {
    const dim3 grid(unsigned(P), unsigned(a.Hkv), unsigned(a.B * a.Tq));
    switch (a.Hq / a.Hkv) {
        case 1: hipLaunchKernelGGL((attn_decode_range_kernel<1>), grid, dim3(256), 0, st, da); break;
        case 2: hipLaunchKernelGGL((attn_decode_range_kernel<2>), grid, dim3(256), 0, st, da); break;
        case 4: hipLaunchKernelGGL((attn_decode_range_kernel<4>), grid, dim3(256), 0, st, da); break;
        case 8: hipLaunchKernelGGL((attn_decode_range_kernel<8>), grid, dim3(256), 0, st, da); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, hipStream_t st) {
    const dim3 grid(unsigned(P), unsigned(a.Hkv), unsigned(a.B * a.Tq));
#define MSA_DM(GG)                                                                                                  \
    hipLaunchKernelGGL((attn_decode_mfma_kernel<GG>), grid, dim3(256), 0, st, static_cast<const uint16_t*>(a.Q),     \
                       a.Tq, a.Hq, a.Hkv, static_cast<const uint16_t*>(a.KVmem), a.mem_off, a.mem_rows_cap,       \
                       a.max_rows, static_cast<const uint16_t*>(a.K_local), static_cast<const uint16_t*>(a.V_local), \
                       a.L, a.q_offset, a.scale * kLog2eD, a.rope_cs, a.max_pos, P, nc, part_o, part_ml)
    switch (a.Hq / a.Hkv) {
        case 1: MSA_DM(1); break;
        case 2: MSA_DM(2); break;
        case 4: MSA_DM(4); break;
        case 8: MSA_DM(8); break;
        default: return hipErrorInvalidValue;
    }
#undef MSA_DM
    return hipGetLastError();
}

hipError_t launch_decode_mfma_mem(const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, int p_base,
                                  int P_total, hipStream_t st) {
    return launch_range(a, decode_args(a, kKeysMem, part_o, part_ml, nc, p_base, P_total), P, st);
}

hipError_t launch_gather_local_attn(const GatherCopyArgs& gc, bool one, int attn_rows, int n_copy,
                                    const AttnArgs& a, float* part_o, float2* part_ml, int P, int nc, int P_total,
                                    hipStream_t st) {
    const DecodeArgs da = decode_args(a, kKeysLocal, part_o, part_ml, nc, 0, P_total);
    const int64_t n_attn = int64_t(P) * a.Hkv * a.B * a.Tq;
    const unsigned grid = unsigned(n_attn + n_copy);
    const int copy_first = one ? int(n_attn) : 0;
#define MSA_GLA(GG)                                                                                              \
    do {                                                                                                         \
        if (one)                                                                                                 \
            hipLaunchKernelGGL((gather_local_attn_kernel<GG, true>), dim3(grid), dim3(256), 0, st, gc, da, P,   \
                               copy_first, n_copy, attn_rows);                                                 \
        else                                                                                                     \
            hipLaunchKernelGGL((gather_local_attn_kernel<GG, false>), dim3(grid), dim3(256), 0, st, gc, da, P,  \
                               copy_first, n_copy, 0);                                                          \
    } while (0)
    switch (a.Hq / a.Hkv) {
        case 1: MSA_GLA(1); break;
        case 2: MSA_GLA(2); break;
        case 4: MSA_GLA(4); break;
        case 8: MSA_GLA(8); break;
        default: return hipErrorInvalidValue;
    }
#undef MSA_GLA
    return hipGetLastError();
}

}  // namespace msa
