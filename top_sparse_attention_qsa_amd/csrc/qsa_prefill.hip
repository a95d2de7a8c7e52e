// QSA sparse-attention prefill for MI355X (gfx950, CDNA4, wave64).
//
// Operation: "Qwen4-Exp QSA llega al Ascend de Huawei" (orcarouter.ai, Spanish
// page), section "Lo que realmente añade la pull request" -- per query token t
// and query head h, softmax(scale * q . K_sel^T) . V_sel over the positions an
// indexer selected for (t, KV head of h); -1 slots masked, an empty row gives
// zero. Positions above t are masked too (causal prefill).
//
// Work decomposition. One wavefront owns one work item (g, t, head chunk):
// the G = Hq/Hkv query heads of KV head g (at most 16 per chunk) against the K
// selected slots of (t, g). Items are independent, so waves never synchronise
// with each other; a block is WPB such waves, two blocks per CU (one for
// caches of 80K rows or more with 32K items or more, see the launch; split
// lists use one-wave blocks). Items are numbered KV-head
// major, and blocks are renumbered so that each XCD (block b runs on XCD
// b % 8) takes runs of consecutive items: the waves sharing an XCD's L2 hold
// neighbouring query positions of one KV head, whose local windows, sinks
// and nearby picks overlap.
//
// Per wave, the K list is walked in tiles of 16 slots:
//   1. one buffer load brings the tile's indices, lane l holding slot l & 15;
//      slots past K read as 0 (range check) and are masked by position;
//      validity 0 <= s <= t gives a 16-bit mask (ballot);
//   2. the 16 K rows and 16 V rows (512 B each) are gathered row-contiguously:
//      each 16-byte load instruction covers two whole rows, lane l reading
//      chunk l & 31 of row 2i + (l >> 5), so every quad of lanes reads 64
//      contiguous bytes and the vector L1 sees whole-line accesses (the row
//      offsets reach the lanes by DPP row broadcasts, or by readlane for
//      micro-block lists). A masked slot gets a
//      byte offset past the end of the buffer: the range check returns zeros
//      and nothing is fetched. The tile goes to registers, then to two padded
//      LDS tiles (K and V), from which the MFMA operands are read in their
//      own layouts;
//   3. S^T = K_tile . Q_g^T on v_mfma_f32_16x16x32_bf16: keys are the M side,
//      the head group (zero-padded to 16) is N, d = 256 is the contraction.
//      Q lives in registers for the whole item;
//   4. online softmax in fp32, base 2. In the S^T layout a lane holds 4 keys
//      of one head. The reference max only moves when some logit exceeds it
//      by a slack of 2^8, so rescaling the accumulators is rare: each lane
//      tests its 4 keys and a ballot decides; only then is the head's max
//      over its 16 keys taken (in-lane max plus two lane-swap steps,
//      v_permlane16_swap / v_permlane32_swap). The row sums stay per lane
//      until the epilogue;
//   5. O^T += V_tile^T . P^T on v_mfma_f32_16x16x32_bf16: V^T comes out of
//      LDS with ds_read_b64_tr_b16 (a 4x16 bf16 block transposed across 16
//      lanes); P^T is already in the B-operand layout. Each weight is sent as
//      a hi + lo pair of bf16 values, contracted in the same MFMA against the
//      V values repeated along k, so the weights carry ~16 significant bits
//      into the fp32 accumulator;
//   6. epilogue: O / l rounded to bf16 (RNE), lse = ln 2 * (m + log2 l); an
//      empty row writes +0.0 and -inf.
// Software pipeline: iteration j stores K of tile j and V of tile j-1 to LDS
// (one store and one new load per pair of rows, so the loads of K of tile
// j+1 and V of tile j go out spread over the stores rather than as a burst
// that would fill the texture unit's queues), then issues the score MFMAs of
// tile j and finishes tile j-1; the two are independent, so the MFMAs run
// under the softmax. Indices run three tiles ahead of the scores; in pool
// form the positions of the listed slots run two tiles ahead, so that a slot
// its position masks (free, or holding a later token) is never gathered.
//
// Split lists (decode). With one query per request there are too few items
// to fill the chip, so each item's list can be cut into n_splits ranges of
// whole tiles, one wave per range. Such a wave writes its unnormalised fp32
// O, its reference max m and its two weight sums to a workspace instead of
// the epilogue, and qsa_combine_kernel merges the ranges of each (row, head):
// with M = max m_s, O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, and lse
// from the fp32 sums likewise.
//
// LDS layout. K tile rows are padded to 528 bytes and V tile rows to 544, so
// consecutive rows start 4 (K) or 8 (V) banks apart and every LDS address is a
// per-lane base plus an immediate. The V tile's stores and transposed reads
// are free of bank conflicts; the K tile's accesses are not entirely (about
// 14% of LDS-active cycles), but an XOR-swizzled K tile without conflicts ran
// no faster.

#include "qsa_internal.h"

#include <math.h>

#include <atomic>
#include <mutex>

namespace qsa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kD = 256;
constexpr int kRowBytes = 512;              // one head's K or V row
constexpr int kNK = 16;                     // selected slots per tile
constexpr int kKStride = kRowBytes + 16;    // LDS row stride of the K tile
constexpr int kVStride = kRowBytes + 32;    // LDS row stride of the V tile
constexpr uint32_t kOob = 0x80000000u;      // byte offset beyond every K/V buffer
constexpr uint32_t kRsrcFlags = 0x00020000u; // raw buffer, 32-bit data format (gfx9)
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleSlack = 8.f;         // log2 headroom before the running max moves

struct KParams {
    const uint16_t *q;
    const uint8_t *k;
    const uint8_t *v;
    const int32_t *idx;
    const int32_t *q_pos;    // pool mode: position of each query row
    const int32_t *slot_pos; // pool mode: position of the token held by each slot
    uint16_t *out;
    float *lse;
    int64_t q_pos0;     // position of query row 0 (sequence modes)
    int32_t n_items;    // Hkv * T * n_hchunks
    int32_t T, Hq, Hkv, G, n_hchunks;
    int32_t K_idx;      // entries per index list
    int32_t K_slots;    // token slots per list: K_idx << blk_shift
    int32_t blk_shift;  // log2 of the tokens named by one entry
    uint32_t n_rows;    // K/V rows (tokens or pool slots)
    uint32_t kv_bytes;  // n_rows * Hkv * 512
    float scale_log2;   // scale * log2(e)
    int32_t n_splits;        // ranges per list (1: no split)
    int32_t tiles_per_split; // tiles per range
    float *ws_o;             // split: fp32 [T, Hq, n_splits, 256] partial O
    f32x4_t *ws_ml;          // split: [T, Hq, n_splits] (m, l, le, 0)
};

// Blocks are dealt round-robin over the 8 XCDs (block b runs on XCD b % 8).
// Renumber in groups of 8 * kXcdChunk blocks (2,048 query rows at 4 items per
// block), cut into 16 pieces of kXcdChunk / 2 consecutive item blocks (128
// rows): XCD x takes piece x, then piece 15 - x. Neighbouring query positions
// then share their window and sink rows in that XCD's L2, all XCDs move
// through the rows together and draw on the same part of the cache at the same
// time, and the cheap rows at the start of each list's ramp (rows below the
// list length, which select fewer slots) are shared evenly: with one piece per
// XCD, the XCD holding the first rows of a group ran out of work early.
// Measured against one 256-row piece per XCD: 1.2-2.1% faster on the
// T = 32,768 and 235K-token workloads, bit-identical results; 64-row pieces
// (four per XCD) were 15% slower (less L2 reuse), one contiguous range per
// XCD 7-8% slower and plain round-robin 20% slower. Blocks past the last whole
// group keep their number.
constexpr uint32_t kXcdChunk = 64;
__device__ __forceinline__ uint32_t xcd_chunked(uint32_t b, uint32_t nb) {
    constexpr uint32_t kPiece = kXcdChunk / 2;
    const uint32_t full = nb / (8 * kXcdChunk) * (8 * kXcdChunk);
    if (b >= full) return b;
    const uint32_t g = b / (8 * kXcdChunk), bl = b % (8 * kXcdChunk);
    const uint32_t x = bl & 7u, i = bl >> 3; // XCD, and the block's rank on it
    const uint32_t piece = i < kPiece ? x : 15u - x;
    return g * 8 * kXcdChunk + piece * kPiece + (i & (kPiece - 1));
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows
// that hold one head) with the gfx950 lane-swap instructions. Swapping a value
// with a copy of itself leaves x[l] in one register and x[l ^ 16] (or
// x[l ^ 32]) in the other. The swap is written out as an instruction with two
// read-write VGPR operands (no memory access) because the compiler treats the
// two results of the builtin with equal operands as equal.
__device__ __forceinline__ void swap_rows16(uint32_t &x, uint32_t &y) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void swap_rows32(uint32_t &x, uint32_t &y) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}

__device__ __forceinline__ float wave_max_across_groups(float v) {
    uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
    swap_rows16(x, y);
    v = fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
    x = __builtin_bit_cast(uint32_t, v);
    y = x;
    swap_rows32(x, y);
    return fmaxf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y));
}

__device__ __forceinline__ float wave_sum_across_groups(float v) {
    uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
    swap_rows16(x, y);
    v = __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
    x = __builtin_bit_cast(uint32_t, v);
    y = x;
    swap_rows32(x, y);
    return __builtin_bit_cast(float, x) + __builtin_bit_cast(float, y);
}

// Indices of one tile: lane l covers token slot j*16 + (l & 15), whose list
// entry is (j*16 + (l & 15)) >> blk_shift (an entry names 2^blk_shift
// consecutive tokens). Entries past the list read as 0 (buffer range check)
// and are masked by slot number.
__device__ __forceinline__ int32_t load_tile_idx(__amdgpu_buffer_rsrc_t ri, int j, int blk_shift, int lane) {
    return __builtin_amdgcn_raw_buffer_load_b32(ri, (uint32_t)((j * kNK + (lane & 15)) >> blk_shift) * 4u, 0, 0);
}

// DPP row_newbcast:N (gfx90a and later): lane N of each 16-lane row is
// broadcast to the whole row.
template <int N>
__device__ __forceinline__ uint32_t row_bcast(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x150 + N, 0xF, 0xF, false);
}

// Byte offsets of the 8 row-pair loads of one tile. Load i covers rows 2i and
// 2i+1: lane l reads 16-byte chunk l & 31 of row 2i + (l >> 5). `off` holds,
// in every lane l, the byte offset of key row l & 15 (kOob when masked).
// Rows 2 and 3 of the wave (lanes 32..63) first take their right neighbour's
// offset (row_shl:1), so one row broadcast of lane 2i gives row 2i to lanes
// 0..31 and row 2i+1 to lanes 32..63; the chunk offset is added in the same
// DPP instruction.
struct TileOffsets {
    uint32_t o[8];
};
template <bool kReadlane>
__device__ __forceinline__ TileOffsets tile_offsets(uint32_t off, int lane) {
    if constexpr (kReadlane) {
        // the same offsets through scalar registers: slower to form, but the
        // loads that use them then go out paced by that work, which the
        // micro-block gather (runs of 4 neighbouring rows) prefers
        const bool upper = (lane >> 5) != 0;
        const uint32_t ch = (uint32_t)(lane & 31) << 4;
        TileOffsets t;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t o0 = __builtin_amdgcn_readlane(off, 2 * i);
            const uint32_t o1 = __builtin_amdgcn_readlane(off, 2 * i + 1);
            t.o[i] = (upper ? o1 : o0) + ch;
        }
        return t;
    }
    const uint32_t ch = (uint32_t)(lane & 31) << 4;
    const uint32_t off2 = (uint32_t)__builtin_amdgcn_update_dpp((int)off, (int)off, 0x101, 0xC, 0xF, false);
    TileOffsets t;
    t.o[0] = row_bcast<0>(off2) + ch;
    t.o[1] = row_bcast<2>(off2) + ch;
    t.o[2] = row_bcast<4>(off2) + ch;
    t.o[3] = row_bcast<6>(off2) + ch;
    t.o[4] = row_bcast<8>(off2) + ch;
    t.o[5] = row_bcast<10>(off2) + ch;
    t.o[6] = row_bcast<12>(off2) + ch;
    t.o[7] = row_bcast<14>(off2) + ch;
    return t;
}
// K of tile j goes to LDS while K of tile j+1 is requested; V of tile j-1
// goes to LDS while V of tile j is requested (a store and a load per pair of
// rows, so the loads are spread out).
__device__ __forceinline__ void rotate_tiles(uint8_t *lk, uint8_t *lv, __amdgpu_buffer_rsrc_t rk,
                                             __amdgpu_buffer_rsrc_t rv, const TileOffsets &tk,
                                             const TileOffsets &tv, u32x4_t (&ks)[8], u32x4_t (&vs)[8],
                                             int lane) {
    const int half = lane >> 5;
    const int c = lane & 31;
    uint8_t *kb = lk + half * kKStride + c * 16;
    uint8_t *vb = lv + half * kVStride + c * 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        *(u32x4_t *)(kb + 2 * i * kKStride) = ks[i];
        ks[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, tk.o[i], 0, 0);
        *(u32x4_t *)(vb + 2 * i * kVStride) = vs[i];
        vs[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, tv.o[i], 0, 0);
    }
}

struct SoftmaxState {
    float m;   // reference max of the base-2 logits (same in every lane of a head)
    float l;   // this lane's share of the sum of the weights as fed to the MFMA
    float le;  // this lane's share of the sum of the fp32 weights (for lse)
};


// Scores of one 16-key tile: S^T[key][head], lane (jg, hl) getting keys
// jg*4 + r (r = 0..3) of head hl.
__device__ __forceinline__ f32x4_t tile_scores(const uint8_t *lk, const bf16x8_t (&qb)[8], int lane) {
    const int hl = lane & 15;
    const int jg = lane >> 4;
    const uint8_t *krow = lk + hl * kKStride + jg * 16;
    // two independent accumulation chains (even and odd d-chunks)
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
        const bf16x8_t a0 = *(const bf16x8_t *)(krow + c * 64);
        const bf16x8_t a1 = *(const bf16x8_t *)(krow + c * 64 + 64);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb[c], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb[c + 1], s1, 0, 0, 0);
    }
    const f32x4_t s = s0 + s1;
    return s;
}

// Online softmax and weighted values of one 16-key tile whose V is in LDS.
__device__ __forceinline__ void tile_finish(f32x4_t s, const uint8_t *lv, uint32_t mask,
                                            f32x4_t (&o)[16], SoftmaxState &st, float scale_log2,
                                            int lane) {
    const int hl = lane & 15;
    const int jg = lane >> 4;

    float x[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        x[r] = ((mask >> (jg * 4 + r)) & 1u) ? s[r] * scale_log2 : -INFINITY;
        lmax = fmaxf(lmax, x[r]);
    }
    // The reference max only moves when some key's logit exceeds it by more
    // than kRescaleSlack (base-2 units): weights stay below 2^kRescaleSlack
    // and the O/l rescale is rare. The test needs only this lane's 4 keys and
    // a ballot; the head's max over its 16 keys (four lanes) is taken only
    // when the rescale happens. The tile has at least one valid key (the
    // caller skips empty tiles), so that max is finite for every head.
    if (__ballot(lmax > st.m + kRescaleSlack)) {
        const float tmax = wave_max_across_groups(lmax);
        const float m_new = fmaxf(st.m, tmax);
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new); // 0 on the first tile
        st.l *= alpha;
        st.le *= alpha;
        st.m = m_new;
#pragma unroll
        for (int db = 0; db < 16; ++db) o[db] *= alpha;
    }

    // Each weight goes to the MFMA as hi + lo, two bf16 values (~16
    // significant bits). The output is normalised by the sum of exactly the
    // values fed to the MFMA (a convex combination of V rows whatever the
    // rounding); lse uses the fp32 sum.
    bf16x4_t pb;
    bf16x4_t pl;
    float psum = 0.f, esum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float pe = __builtin_amdgcn_exp2f(x[r] - st.m);
        const __bf16 hi = (__bf16)pe;
        const __bf16 lo = (__bf16)(pe - (float)hi);
        pb[r] = hi;
        pl[r] = lo;
        esum += pe;
        psum += (float)hi + (float)lo;
    }
    st.l += psum;
    st.le += esum;

    // V^T operand: lane (jg, hl) addresses row jg*4 + (hl >> 2), 8 bytes at
    // d = db*16 + (hl & 3)*4; the transposed read returns column d = db*16 + hl
    // of rows jg*4 + 0..3. One 16x16x32 MFMA per d-block contracts both
    // weight halves at once: the V^T values are repeated along k, the B
    // operand carries P_hi for the first four k and P_lo for the last four.
    const int R = jg * 4 + (hl >> 2);
    const uint8_t *vrow = lv + R * kVStride + (hl & 3) * 8;
    const bf16x8_t pp = {pb[0], pb[1], pb[2], pb[3], pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
    for (int db = 0; db < 16; ++db) {
        const bf16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(vrow + db * 32));
        const bf16x8_t vv = {va[0], va[1], va[2], va[3], va[0], va[1], va[2], va[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pp, o[db], 0, 0, 0);
    }
}

// Index forms (kMode):
//   kTokens  entries are token positions; a token s is used iff
//            0 <= s <= q_pos0 + row;
//   kBlocks  an entry b names tokens b << blk_shift .. +2^blk_shift - 1, each
//            used under the same rule;
//   kPool    entries are slots of a K/V pool; slot s is used iff
//            0 <= s < n_rows and 0 <= slot_pos[s] <= q_pos[row].
// In every form a slot that is not used gets no row offset: its K/V row is
// never read, whatever it holds.
enum IndexForm { kTokens = 0, kBlocks = 1, kPool = 2 };

template <int WPB, int kMode, bool kSplit>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(2, 2))) void qsa_prefill_kernel(const KParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_k[WPB][kNK * kKStride];
    __shared__ __attribute__((aligned(16))) uint8_t lds_v[WPB][kNK * kVStride];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t item = (int32_t)xcd_chunked(blockIdx.x, gridDim.x) * WPB + w;
    if (item >= p.n_items) return;

    const int32_t sp = kSplit ? item % p.n_splits : 0;
    const int32_t item_h = kSplit ? item / p.n_splits : item;
    const int32_t hc = item_h % p.n_hchunks;
    const int32_t rest = item_h / p.n_hchunks;
    const int32_t row = rest % p.T;
    const int32_t g = rest / p.T;
    constexpr bool kIsPool = kMode == kPool;
    // measured per index form: micro-block lists run 8% faster with the row
    // offsets formed through readlane, token lists 1% faster with DPP
    constexpr bool kRlOffsets = kMode == kBlocks;
    // absolute position of this query
    const int64_t tq = kIsPool ? (int64_t)p.q_pos[row] : p.q_pos0 + row;
    const int h0 = g * p.G + hc * 16;
    const int nh = min(16, p.G - hc * 16);
    const int hl = lane & 15;
    const int jg = lane >> 4;

    // Q group as the B operand: lane (jg, hl) holds head hl, d = c*32 + jg*8 .. +8.
    bf16x8_t qb[8];
    if (hl < nh) {
        const uint16_t *qrow = p.q + ((int64_t)row * p.Hq + h0 + hl) * kD + jg * 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) qb[c] = *(const bf16x8_t *)(qrow + c * 32);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            for (int e = 0; e < 8; ++e) qb[c][e] = (__bf16)0.f;
    }

    f32x4_t o[16];
#pragma unroll
    for (int db = 0; db < 16; ++db) o[db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    SoftmaxState st = {-INFINITY, 0.f, 0.f};

    // this wave's tiles: [j_begin, j_end) of the list
    const int n_list_tiles = (p.K_slots + kNK - 1) / kNK;
    const int j_begin = kSplit ? sp * p.tiles_per_split : 0;
    const int j_end = kSplit ? min(n_list_tiles, j_begin + p.tiles_per_split) : n_list_tiles;
    const int32_t slot_end = min(p.K_slots, j_end * kNK);
    if (j_end > j_begin) {
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)p.k, 0, (int)p.kv_bytes, kRsrcFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)p.v, 0, (int)p.kv_bytes, kRsrcFlags);
        const int32_t *irow = p.idx + ((int64_t)row * p.Hkv + g) * p.K_idx;
        const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc((void *)irow, 0, p.K_idx * 4, kRsrcFlags);
        __amdgpu_buffer_rsrc_t rp = ri;
        if constexpr (kIsPool)
            rp = __builtin_amdgcn_make_buffer_rsrc((void *)p.slot_pos, 0, (int)(p.n_rows * 4u), kRsrcFlags);
        const uint32_t row_stride = (uint32_t)p.Hkv * kRowBytes;
        const uint32_t head_off = (uint32_t)g * kRowBytes;
        const int shift = kMode == kBlocks ? p.blk_shift : 0;
        const int32_t sub = hl & ((1 << shift) - 1);
        const int32_t bmax = INT32_MAX >> shift;
        uint8_t *lk = &lds_k[w][0];
        uint8_t *lv = &lds_v[w][0];

        // Pool form: the position of the token held by pool slot e (read as 0
        // for an entry outside the pool, which the slot test masks anyway).
        // It is loaded one iteration before the slot's tile forms its row
        // offsets, so a slot that its position masks (a free slot, a token
        // after the query) is never gathered: its row may hold anything,
        // NaN included, and contributes nothing.
        auto load_spos = [&](int32_t e) -> int32_t {
            if constexpr (kIsPool) {
                const bool in_pool = e >= 0 && (uint32_t)e < p.n_rows;
                return __builtin_amdgcn_raw_buffer_load_b32(rp, in_pool ? (uint32_t)e * 4u : kOob, 0, 0);
            } else {
                return 0;
            }
        };
        // Row byte offset of this lane's slot in tile j, entry e (pool form:
        // slot position spos), or kOob when the slot cannot be used (the range
        // check then returns zeros and fetches nothing); `mask` gets the
        // tile's validity bits (bit k = key k).
        auto prep = [&](int j, int32_t e, int32_t spos, uint32_t &mask) -> uint32_t {
            const bool in_list = j * kNK + hl < slot_end;
            bool ok;
            uint32_t off;
            if constexpr (kIsPool) {
                ok = in_list && e >= 0 && (uint32_t)e < p.n_rows && spos >= 0 && (int64_t)spos <= tq;
                off = (uint32_t)e * row_stride + head_off;
            } else {
                const int32_t s = (int32_t)(((uint32_t)e << shift) | (uint32_t)sub); // used only if e <= bmax
                ok = in_list && e >= 0 && e <= bmax && (int64_t)s <= tq;
                off = (uint32_t)s * row_stride + head_off;
            }
            mask = (uint32_t)__ballot(ok) & 0xFFFFu;
            return ok ? off : kOob;
        };

        // Software pipeline, one tile deep: iteration j writes K of tile j
        // and V of tile j-1 to LDS, requests K of tile j+1 and V of tile j,
        // then computes the scores of tile j and finishes tile j-1 (softmax,
        // weighted values). The two halves are independent, so the MFMAs of
        // one overlap the vector work of the other. Loads past the range are
        // masked (nothing fetched); the loop runs one iteration past the last
        // tile to finish it. Pool slot positions run two tiles ahead.
        u32x4_t ks[8], vs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) vs[i] = (u32x4_t){0u, 0u, 0u, 0u};
        int32_t i0 = load_tile_idx(ri, j_begin, shift, lane);
        int32_t inext = load_tile_idx(ri, j_begin + 1, shift, lane);
        const int32_t sp0 = load_spos(i0);
        int32_t sp_next = load_spos(inext);
        uint32_t mask_cur;
        uint32_t off_cur = prep(j_begin, i0, sp0, mask_cur);
        {
            const TileOffsets t0 = tile_offsets<kRlOffsets>(off_cur, lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) ks[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, t0.o[i], 0, 0);
        }
        int32_t inext2 = load_tile_idx(ri, j_begin + 2, shift, lane);
        f32x4_t s_prev = {0.f, 0.f, 0.f, 0.f};
        uint32_t mask_prev = 0;
        for (int j = j_begin;; ++j) {
            uint32_t mask_next;
            const uint32_t off_next = prep(j + 1, inext, sp_next, mask_next);
            sp_next = load_spos(inext2); // tile j+2
            rotate_tiles(lk, lv, rk, rv, tile_offsets<kRlOffsets>(off_next, lane),
                         tile_offsets<kRlOffsets>(off_cur, lane), ks, vs, lane);
            inext = inext2;
            inext2 = load_tile_idx(ri, j + 3, shift, lane);
            const f32x4_t sc = tile_scores(lk, qb, lane);
            if (mask_prev) tile_finish(s_prev, lv, mask_prev, o, st, p.scale_log2, lane);
            if (j >= j_end) break;
            s_prev = sc;
            mask_prev = mask_cur;
            mask_cur = mask_next;
            off_cur = off_next;
        }
    }

    const float l_tot = wave_sum_across_groups(st.l);
    const float le_tot = wave_sum_across_groups(st.le);
    if constexpr (kSplit) {
        // partial of range sp: O relative to 2^m, lane (jg, hl) holding
        // d = db*16 + jg*4 + r of head h0 + hl
        if (hl < nh) {
            const int64_t prow = ((int64_t)row * p.Hq + h0 + hl) * p.n_splits + sp;
            float *wo = p.ws_o + prow * kD + jg * 4;
#pragma unroll
            for (int db = 0; db < 16; ++db) *(f32x4_t *)(wo + db * 16) = o[db];
            if (jg == 0) p.ws_ml[prow] = (f32x4_t){st.m, l_tot, le_tot, 0.f};
        }
        return;
    }
    if (hl < nh) {
        const int64_t orow = (int64_t)row * p.Hq + h0 + hl;
        uint16_t *optr = p.out + orow * kD + jg * 4;
        const bool empty = !(l_tot > 0.f);
        const float inv = empty ? 0.f : 1.0f / l_tot;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
            bf16x4_t r4;
#pragma unroll
            for (int r = 0; r < 4; ++r) r4[r] = (__bf16)(o[db][r] * inv);
            *(bf16x4_t *)(optr + db * 16) = r4;
        }
        if (jg == 0) p.lse[orow] = empty ? -INFINITY : (st.m + __log2f(le_tot)) * kLn2;
    }
}

// Merge of the n_splits partials of each (row, head): one wave per pair,
// lane l owning d = 4l .. 4l+3. Up to 16 ranges are taken per round: their
// (m, l, le) records and partial rows are all requested before any is used,
// then folded into a running result whose reference max M moves when a
// round's max exceeds it. A range with no valid key has m = -inf and weight
// 0; a row with none at all gets +0.0 and lse = -inf.
template <int WPB>
__global__ __launch_bounds__(64 * WPB) void qsa_combine_kernel(const float *__restrict__ ws_o,
                                                               const f32x4_t *__restrict__ ws_ml,
                                                               uint16_t *__restrict__ out, float *__restrict__ lse,
                                                               int32_t n_pairs, int32_t n_splits) {
    constexpr int kRound = 16;
    const int lane = threadIdx.x & 63;
    const int32_t pair = (int32_t)blockIdx.x * WPB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (pair >= n_pairs) return;
    const f32x4_t *ml = ws_ml + (int64_t)pair * n_splits;
    const float *po = ws_o + (int64_t)pair * n_splits * kD + lane * 4;

    float M = -INFINITY, L = 0.f, LE = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < n_splits; s0 += kRound) {
        const int n = min(kRound, n_splits - s0);
        f32x4_t rec[kRound], part[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            if (u < n) {
                rec[u] = ml[s0 + u];
                part[u] = *(const f32x4_t *)(po + (int64_t)(s0 + u) * kD);
            } else {
                rec[u] = (f32x4_t){-INFINITY, 0.f, 0.f, 0.f};
                part[u] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            }
        }
        float cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < kRound; ++u) cm = fmaxf(cm, rec[u][0]);
        const float Mn = fmaxf(M, cm);
        if (Mn == -INFINITY) continue;
        const float a = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        acc *= a;
        L *= a;
        LE *= a;
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const float w = rec[u][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(rec[u][0] - Mn);
            acc += w * part[u];
            L += w * rec[u][1];
            LE += w * rec[u][2];
        }
        M = Mn;
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.0f / L;
    bf16x4_t r4;
#pragma unroll
    for (int r = 0; r < 4; ++r) r4[r] = (__bf16)(acc[r] * inv);
    *(bf16x4_t *)(out + (int64_t)pair * kD + lane * 4) = r4;
    if (lane == 0) lse[pair] = empty ? -INFINITY : (M + __log2f(LE)) * kLn2;
}

// Occupancy by cache length and work size. Two blocks per CU (8 waves) suit
// caches of up to ~64K rows; from ~80K rows on, one block per CU (4 waves) is
// 5-32% faster once there are at least 32K work items (measured at 82K-235K
// rows with uniform and recency-weighted lists, and on a 246K-slot pool),
// while at 65K rows it is 11% slower to even, and with 8K-16K items against a
// 131K-row cache it is up to 15% slower. The launch reserves extra dynamic LDS
// that the kernel never touches, so that a second block no longer fits in the
// CU's 160 KB.
constexpr uint32_t kOneBlockRows = 81920;
constexpr int32_t kOneBlockItems = 32768;
constexpr size_t kLdsPerCu = 160 * 1024;

template <int WPB, int kMode, bool kSplit>
qsa_status_t launch(const KParams &kp, hipStream_t stream) {
    const uint32_t blocks = (uint32_t)((kp.n_items + WPB - 1) / WPB);
    constexpr size_t kLdsPerBlock = (size_t)WPB * kNK * (kKStride + kVStride);
    static_assert(2 * kLdsPerBlock <= kLdsPerCu, "two blocks must fit for the short-cache case");
    const bool one_block = !kSplit && kp.n_rows >= kOneBlockRows && kp.n_items >= kOneBlockItems;
    const size_t pad = one_block ? kLdsPerCu / 2 + 1024 - kLdsPerBlock : 0;
    hipLaunchKernelGGL((qsa_prefill_kernel<WPB, kMode, kSplit>), dim3(blocks), dim3(64 * WPB), pad, stream, kp);
    if (hipGetLastError() != hipSuccess) return QSA_ERR_LAUNCH;
    if constexpr (kSplit) {
        const int32_t n_pairs = kp.T * kp.Hq;
        hipLaunchKernelGGL((qsa_combine_kernel<4>), dim3((uint32_t)((n_pairs + 3) / 4)), dim3(256), 0, stream,
                           (const float *)kp.ws_o, (const f32x4_t *)kp.ws_ml, kp.out, kp.lse, n_pairs, kp.n_splits);
        if (hipGetLastError() != hipSuccess) return QSA_ERR_LAUNCH;
    }
    return QSA_OK;
}

} // namespace

qsa_status_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    KParams kp;
    kp.q = (const uint16_t *)a.q;
    kp.k = (const uint8_t *)a.k;
    kp.v = (const uint8_t *)a.v;
    kp.idx = a.idx;
    kp.q_pos = a.q_pos;
    kp.slot_pos = a.slot_pos;
    kp.out = (uint16_t *)a.out;
    kp.lse = a.lse;
    kp.q_pos0 = a.q_pos0;
    kp.T = (int32_t)a.T;
    kp.Hq = a.Hq;
    kp.Hkv = a.Hkv;
    kp.G = a.Hq / a.Hkv;
    kp.n_hchunks = (int32_t)(((int64_t)kp.G + 15) / 16);
    kp.K_idx = a.K;
    kp.blk_shift = a.blk_shift;
    kp.K_slots = a.K << a.blk_shift;
    const int64_t n_items = a.T * a.Hkv * kp.n_hchunks;
    if (n_items > INT32_MAX - 4) return QSA_ERR_UNSUPPORTED;
    kp.n_items = (int32_t)n_items;
    kp.n_rows = (uint32_t)a.n_kv_rows;
    kp.kv_bytes = (uint32_t)(a.n_kv_rows * a.Hkv * kRowBytes);
    kp.scale_log2 = a.scale * 1.44269504088896340736f;
    kp.n_splits = 1;
    kp.tiles_per_split = 0;
    kp.ws_o = nullptr;
    kp.ws_ml = nullptr;
    if (a.n_splits > 1) {
        // pool form only (decode); workspace: [pairs * n_splits] (m, l, le, 0)
        // records, then [pairs * n_splits * 256] fp32 partial O
        if (!a.pool || a.workspace == nullptr) return QSA_ERR_INVALID_ARG;
        const int64_t split_items = n_items * a.n_splits;
        if (split_items > INT32_MAX - 4) return QSA_ERR_UNSUPPORTED;
        kp.n_items = (int32_t)split_items;
        kp.n_splits = a.n_splits;
        kp.tiles_per_split = a.tiles_per_split;
        kp.ws_ml = (f32x4_t *)a.workspace;
        kp.ws_o = (float *)((f32x4_t *)a.workspace + a.T * a.Hq * a.n_splits);
        // one wave per block: the ~512 range waves then spread over all 256 CUs
        // (with 4-wave blocks they filled half of them; 1-wave blocks are 5%
        // faster per decode step)
        return launch<1, kPool, true>(kp, stream);
    }
    if (a.pool) return launch<4, kPool, false>(kp, stream);
    return a.blk_shift ? launch<4, kBlocks, false>(kp, stream) : launch<4, kTokens, false>(kp, stream);
}

} // namespace qsa

// Scratch of qsa_sparse_decode_noalloc: the split partials of one decode call
// ((m, l, le) records, then fp32 partial rows), in device memory that the
// library holds from its load until the process ends, one copy per GPU. In
// host code `scratch` names a host-side stand-in, not device memory: kernels
// and copies get the address from device_scratch below.
static __device__ __align__(256) uint8_t scratch[QSA_DECODE_SCRATCH_BYTES];

namespace qsa {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;
} // namespace

qsa_status_t device_scratch(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return QSA_ERR_LAUNCH;
    if (dev >= kMaxDevices) return QSA_ERR_UNSUPPORTED;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // with device `dev` current: that device's copy of the array
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError(); // do not leave the error for the caller's next HIP call
                return QSA_ERR_LAUNCH;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return QSA_OK;
}

} // namespace qsa
