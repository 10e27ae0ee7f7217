// Decode attention core for the DeepSeek-V2 geometry (n_h = 128, d_c = 512,
// d_r = 64, bf16 cache), on gfx950 MFMA.
//
// What it computes (order B of the walkthrough's §3, "顺序 B"): for each head
// i and cached row j = [c^KV_j | k^R_j] (576 bf16 numbers, no head index, the
// walkthrough's step 1), the score s_ij = Q~_i . row_j with the absorbed query
// Q~_i = [W_UK,i^T q^C_i | q^R_i] * scale, a softmax over j, and the weighted
// sum of the latents o~_i = sum_j p_ij c^KV_j in 512-d latent space.
//
// Design (gfx950):
//  * one work-group per compute unit (4 waves, one per SIMD).  For the scores
//    wave w owns heads [32w, 32w+32) and keeps their whole absorbed query in
//    registers (36 x 16 B per lane).  For the latent accumulation it owns
//    latent dims [128w, 128w+128) of all 128 heads: a 128 x 128 fp32
//    accumulator that fills the 256 accumulation registers.  The waves swap
//    their softmax numerators P through LDS, so each wave reads only its
//    quarter of the latent tile for the second contraction.
//  * with one wave per SIMD the instruction stream sets the pace: beside each
//    32-cycle MFMA there is room for about four other instructions before the
//    MFMA pipe idles.  So every LDS read is a per-lane base register plus an
//    immediate offset (one XOR-derived base per four score reads, two for
//    the accumulation reads, moved with the ring slot once per sub-tile), the
//    cache operand of the second contraction comes straight from
//    ds_read_b64_tr_b16 (no register shuffles), the softmax is an exp2 and a
//    pack per score in one branch-free block beside the accumulation MFMAs,
//    and the scalar set-up of the next sub-tile's ring loads is formed in
//    the shadow of the current sub-tile's score MFMAs.
//  * 32-token sub-tiles stream through a four-slot LDS ring with 16-byte
//    direct-to-LDS buffer loads, two sub-tiles in flight while the scores of
//    sub-tile j and the accumulation of sub-tile j-1 run.  A slot holds the
//    32 latent parts (1024 B each) and then the 32 RoPE parts (128 B each);
//    16-byte pieces are XOR-permuted per row so that every LDS read pattern
//    below is free of bank conflicts, and each ring load covers exactly one
//    row's latent part (or the RoPE parts of eight rows), which keeps its
//    address arithmetic to one or two instructions.  A descriptor's range is
//    the sub-tile's valid rows, so a partial sub-tile needs no clamping: the
//    rows past it arrive as zeros.
//  * scores: S^T[token][head] = C[token][dims] . Q~^T[dims][head] with
//    v_mfma_f32_32x32x16_bf16 (A = cache rows from LDS, B = Q~), 36 K-steps.
//    The absorption writes query tiles that carry a factor log2(e), so the
//    scores come out in log2 units; tiles rearranged from a caller's rows
//    are exact copies, and that variant multiplies in the exponent's fma.
//  * softmax numerators 2^s with no reference at all in a first pass (exact
//    softmax algebra while every numerator stays inside fp32/bf16 range), so
//    the 256-register accumulator is never rescaled.  Each head's maximum is
//    tracked; if any head of the work-group ends a segment with its maximum
//    outside [-64, 64], the whole segment is redone once with each head's
//    maximum as the reference (numerators <= 1): after the segment every
//    wave ORs its 32 heads' flags into one vote, and the work-group ORs the
//    four votes through LDS.
//  * latent accumulation: o~^T[dims][head] += C^T[dims][tokens] . P^T.  The
//    token order inside a sub-tile is chosen so that the score registers are
//    P^T's operand as they stand, and each transposing read fetches four
//    tokens four rows apart (conflict-free under the XOR permutation).
//  * the MFMA stream of an iteration interleaves the 36 score steps with the
//    32 accumulation steps and the ring refill; sched_barrier pins the order.
//  * a work-group walks the segments the plan assigns to it and writes each
//    segment's unnormalised (m, l, o~) from the accumulation registers, o~ as
//    bf16 in register order; a merge kernel weighs the segments of each
//    sequence by e^(m_s - M) / sum_s l_s e^(m_s - M) and writes o~ as bf16.
#include <math.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));

constexpr int kHeads = 128;
constexpr int kRow = 576;             // bf16 numbers per cached token
constexpr int kDc = 512;
constexpr int kRowBytes = kRow * 2;   // 1152: one cached row in HBM
constexpr int kSub = 32;              // tokens per sub-tile (one MFMA block)
constexpr int kSlots = 4;             // LDS ring slots
constexpr int kLatBytes = 1024;       // LDS row of the latent part
constexpr int kRopeBytes = 128;       // LDS row of the RoPE part
constexpr int kRopeOff = kSub * kLatBytes;                 // 32768
constexpr int kSubBytes = kRopeOff + kSub * kRopeBytes;    // 36864
constexpr int kPBufBytes = 4 * 2 * 64 * 16;                // [wave][K-step][lane][16 B]
// the two P buffers first (their offsets fit a ds_read immediate), then the
// ring; every slot base is a multiple of 4096, so it never meets the XOR-ed
// address bits 4..7
constexpr int kPBufOff = 0;
constexpr int kRingOff = 2 * kPBufBytes;                   // 16384
constexpr int kLdsBytes = kRingOff + kSlots * kSubBytes;   // 163840 = 160 KB
constexpr int kInstsPerWave = 9;      // ring loads per wave per sub-tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKSteps = kRow / 16;    // 36 score K-steps of 16 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 64.0f;        // largest |head maximum| a pass without reference takes (log2 units)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, gfx9 family

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4bf16 lds_v4bf16;

__device__ __shared__ __attribute__((aligned(16))) char g_lds[kLdsBytes];

// Work-group barrier without __syncthreads' release fence: that fence waits
// for every outstanding vector memory operation, which would drain the
// in-flight cache sub-tiles of the ring at each barrier.  LDS ordering is
// established by the explicit s_waitcnt that precedes each use; the asm
// memory clobbers keep the compiler from moving LDS accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte piece c of a row's RoPE part (8 pieces) sits at position
// c ^ swz_rope(r) of LDS RoPE row r; piece c of the latent part (64 pieces)
// sits at position c ^ (r & 15).
__device__ inline int swz_rope(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

// x ^ c formed at the point of use.  Left to itself the compiler hoists every
// swizzled LDS address of the loop body into its own register for the whole
// loop, which the register budget of the attention kernel cannot afford.
template <int C>
__device__ inline int xor_here(int x) {
  if constexpr (C == 0) {
    return x;
  } else {
    int r;
    asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "i"(C), "v"(x));
    return r;
  }
}

// This lane's index, formed at the point of use.  A lane-derived value kept
// from the kernel's start is live across the sub-tile loop, where the
// register budget spills it, and the spill's reload in a segment's epilogue
// waits for every vector memory operation in flight (vmcnt(0)): the next
// segment's query, its first sub-tiles and the partial stores.
__device__ inline int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// f(integral_constant<int, I>) for I in [I0, N): unrolled with compile-time indices
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
template <int I>
using ic = std::integral_constant<int, I>;

// score MFMAs with a VGPR accumulator (first K-step starts from zero; the
// early clobber keeps its destination off the A/B operands)
__device__ __forceinline__ void score_mfma_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_mfma(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

template <typename T>
__device__ inline T lds_load(int byte) {
  return *(const T __attribute__((address_space(3)))*)((lds_char*)g_lds + byte);
}
template <typename T>
__device__ inline void lds_store(int byte, T v) {
  *(T __attribute__((address_space(3)))*)((lds_char*)g_lds + byte) = v;
}

// One 32-token sub-tile in flight: rows [0, 32) of a page run starting at
// the descriptor's base go to LDS slot `slot`.  The descriptor's range covers
// the sub-tile's nvalid rows only: a lane whose row lies at or past nvalid is
// out of range, reads no memory and writes zeros to LDS (gfx950 range-checks
// the whole offset, soffset included), so those rows hold zeros, whose
// scores are masked to zero weight (0 * 0 never turns into NaN).  Wave w
// moves rows [8w, 8w+8): loads 0..7 the latent part of one row each, load 8
// the RoPE parts of all eight.  Every wave issues exactly kInstsPerWave loads
// per sub-tile whatever nvalid is; the ring's vmcnt bookkeeping relies on it.
//
// The loads are MUBUF direct-to-LDS loads written as inline asm.  The
// compiler's own LDS-DMA tracking would otherwise treat them as possible
// writers of every later LDS read it cannot disambiguate - the transposing
// ds_read_b64_tr_b16 among them - and wait for all vector memory operations
// (vmcnt(0)) before each such read, draining the ring.  The kernel orders
// ring data itself: an explicit vmcnt wait for its own sub-tile, then a
// barrier.  (The loads write no registers, so no register result of an asm
// load is ever left in flight.)
//
// Each cache row is read once per step, so the loads carry the nontemporal
// hint (nt): on the batch-64 workload attention plus merge took 4.6% less
// time with it.  A plain read stream of the cache's size showed the same
// thing, 6.5 TB/s with the hint against 5.9 without.
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct Refill {
  i32x4 rs;   // buffer descriptor (base, valid bytes) in scalar registers
  int slot;   // LDS byte offset of the ring slot
};

// raw buffer descriptor over [p, p + bytes) (uniform values; readfirstlane
// keeps the words scalar where the compiler would hold one in a vector
// register, which the loads' scalar operand cannot take)
__device__ inline i32x4 make_rsrc(const void* p, int bytes) {
  const unsigned long long a = (unsigned long long)p;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(unsigned)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3};
}

__device__ inline void lds_dma16(const i32x4& rs, int voff, int lds_byte) {
  const int m0 = __builtin_amdgcn_readfirstlane(
      (int)(uintptr_t)((lds_char*)g_lds + lds_byte));
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :: "v"(voff), "s"(rs), "s"(m0) : "m0");
}

// lat16: (lane ^ 8 (w & 1)) << 4, the lane's piece position of row 8w (the
// XOR permutation of rows 8w + i differs from it by i); rope_off: this lane's
// source offset in the RoPE load (row 8w + lane / 8).  Each offset carries
// its row, so the range check alone bounds a partial sub-tile.
__device__ inline void ring_load(const Refill& rf, int i, int wave, int lat16, int rope_off) {
  if (i < 8) {
    const int r = 8 * wave + i;
    lds_dma16(rf.rs, (lat16 ^ (i << 4)) + r * kRowBytes, rf.slot + r * kLatBytes);
  } else {
    lds_dma16(rf.rs, rope_off, rf.slot + kRopeOff + 8 * wave * kRopeBytes);
  }
}

// kQLog2e: the query tiles carry log2(e) (written so by the absorption, one
// rounding from fp32); otherwise they are the caller's rows rearranged, and
// each score is scaled by log2(e) inside the exponent's fma.
template <bool kQLog2e>
__global__ __launch_bounds__(kThreads, 1) void attn_v2_kernel(
    const __bf16* __restrict__ q_abs, const __bf16* __restrict__ cache, int num_pages,
    const int32_t* __restrict__ page_table, int max_pages, int page,
    const int* __restrict__ counts, const int* __restrict__ wg_seg_start,
    const Seg* __restrict__ segs, __bf16* __restrict__ part_o, float* __restrict__ part_ml) {
  // Work-groups are dispatched round-robin over the eight XCDs.  Give the
  // work-groups of one XCD consecutive plan slots: consecutive slots share
  // sequences, so a sequence's absorbed query is fetched into one L2.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int g = xcd * (G >> 3) + min(xcd, G & 7) + (blockIdx.x >> 3);
  if (g >= counts[1]) return;
  const int k_begin = wg_seg_start[g];
  const int k_end = wg_seg_start[g + 1];
  if (k_begin >= k_end) return;
  // wave-uniform: a scalar register, so the LDS destinations of the ring
  // loads (M0) are scalar arithmetic rather than per-lane values
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;     // lane half
  const int m32 = lane & 31;

  // ---- per-lane LDS byte offsets, relative to ring slot 0 and moved with
  // the ring slot once per sub-tile (so every read below is a base register
  // plus an immediate offset).
  //
  // Token order.  Score-MFMA row m = 16 kap + 8 b + 4 hm + r (kap, b, hm in
  // {0, 1}, r < 4) reads sub-tile token rho(m) = 16 kap + 4 r + 2 b + hm.  The
  // score registers of lane (head, hm) then hold, in register i = 8 kap + e,
  // the token rho(16 kap + 8 (e / 4) + 4 hm + e % 4) - exactly the K index
  // 16 kap + 8 hm + e of the latent accumulation's operands, so P needs no
  // rearranging; and each transposing LDS read of the accumulation's cache
  // operand fetches four tokens four rows apart, so that the 32 lanes it
  // serves at once hit 16 distinct 16-byte bank groups under the XOR
  // permutation (rows two apart would pair them up).
  const int R = (m32 & 16) + 4 * (m32 & 3) + 2 * ((m32 >> 3) & 1) + ((m32 >> 2) & 1);
  // scores, latent K-step ks = 8 a + b (16 dims): row R, 16-byte piece
  // 2 ks + h at position (2 ks + h) ^ (R & 15) -> (qb ^ 32 b) + 256 a.  The
  // score chain walks b-major (ks = 8 a + b for b = 0..7, a = 0..3), so each
  // XOR-derived base serves four consecutive K-steps.
  int qb = kRingOff + R * kLatBytes + ((h ^ (R & 15)) << 4);
  // scores, RoPE K-step 32 + t: row R, RoPE piece 2 t + h -> qrb ^ (t << 5)
  int qrb = kRingOff + kRopeOff + R * kRopeBytes + ((h ^ swz_rope(R)) << 4);
  // accumulation operand (cache^T: 32 dims x 16 tokens) by ds_read_b64_tr_b16:
  // in each 16-lane group gq, lane 4 rr + jj supplies 4 dims (chunk jj) of
  // token row rr; output lane i then holds dim i of the four rows.  Dims
  // block mb of this wave = dims 128 wave + 32 mb + [0, 32); K-step kap, read
  // bb: token rows 16 kap + 4 rr + 2 bb + h.  Every bit of the position
  // (chunk piece ^ row & 15) pairs a lane bit with mb or bb, so the address
  // of (mb, bb, kap) is (tb ^ (32 bb + 64 mb)) + 1024 (16 kap + 2 bb).
  int tb;
  {
    const int gq = lane >> 4, ii = lane & 15, rr = ii >> 2, jj = ii & 3;
    tb = kRingOff + (4 * rr + h) * kLatBytes +
         ((16 * wave + ((jj >> 1) ^ h) + 2 * (gq & 1) + 4 * (rr & 1) + 8 * (rr >> 1)) << 4) +
         8 * (jj & 1);
  }
  // this lane's 16-byte column of a P buffer block: P of head block n, K-step
  // kap sits at buffer + (2 n + kap) * 1024 + 16 lane
  const int pl = 16 * lane;
  // ring loads: this lane's piece position in row 8 wave, and its source
  // offset in a full sub-tile's RoPE load
  const int lat16 = (lane ^ (8 * (wave & 1))) << 4;
  const int rope_off = (8 * wave + (lane >> 3)) * kRowBytes + kLatBytes +
                       (((lane & 7) ^ swz_rope(8 * wave + (lane >> 3))) << 4);
  int slot_cur = 0;   // ring slot the bases currently point into
  auto move_bases = [&](int slot) {
    const int d = (slot - slot_cur) * kSubBytes;
    slot_cur = slot;
    qb += d;
    qrb += d;
    tb += d;
  };
  auto slot_off = [](int pos) { return kRingOff + (pos & (kSlots - 1)) * kSubBytes; };

  // Page ids, 64 pages per window: lane i holds the id of page w0 + i of
  // sequence b (-1 past the table row).  A vector register instead of scalar
  // loads: an outstanding scalar load would force a full LDS wait
  // (lgkmcnt(0)) at every use of an LDS read in the loop below.
  auto load_window = [&](int b, int w0) {
    const int p = w0 + lane_here();
    return p < max_pages ? page_table[(long)b * max_pages + p] : -1;
  };

  // ---- ring refill cursor.  The work-group's sub-tiles form one stream
  // (segment after segment); ring position pos holds a stream sub-tile in
  // slot pos mod 4.  Each computing iteration consumes one position and loads
  // the one two ahead, so near a segment's end the cursor walks into the
  // next segment and that segment's first sub-tiles arrive while this one is
  // still computed.  Cursor: sequence rb, rrem tokens left, at byte offset
  // rpo_b of page rpi, page window wb / pid; seg_bit marks the cursor's
  // segment in badm.
  int rb = 0, rrem = 0, rpi = 0, rpo_b = 0, wb = 0, pid = 0;
  unsigned seg_bit = 0;
  int k = k_begin;      // the segment being computed
  int pid_next = 0;     // window of segment k + 1's first pages (loaded ahead)
  unsigned badm = 0;    // bit s & 31: segment s met a page id out of range
  // a segment descriptor, waited for here: a scalar load left in flight
  // would turn every later LDS wait of the iteration into lgkmcnt(0)
  auto seg_at = [&](int kk) {
    Seg sg = segs[kk];
    asm volatile("" :: "v"(sg.b), "v"(sg.t0), "v"(sg.t1));
    return sg;
  };
  auto cursor_begin = [&](int kk, int w) {
    const Seg sg = seg_at(kk);
    seg_bit = 1u << (kk & 31);
    rb = sg.b;
    rrem = __builtin_amdgcn_readfirstlane(sg.t1 - sg.t0);   // scalar: a uniform count
    wb = sg.t0 / page;
    rpi = wb;
    rpo_b = (sg.t0 - wb * page) * kRowBytes;
    pid = w;
  };
  // one sub-tile on: the next page after the last one of a page
  auto cursor_step = [&]() {
    rrem -= kSub;
    const bool wrap = rpo_b + kSub * kRowBytes == page * kRowBytes;
    rpo_b = wrap ? 0 : rpo_b + kSub * kRowBytes;
    rpi += wrap ? 1 : 0;
  };
  // the cursor's next sub-tile, for ring position pos (sub-tiles never
  // straddle a page: page is a multiple of 64 and segments start on 64-token
  // boundaries or at 0)
  // The cursor's next sub-tile (rrem > 0), for ring position pos: selects
  // only, no branch but the rare window change.  A page id out of range
  // gives a descriptor of zero bytes and marks the segment.
  auto refill_at = [&](int pos) {
    if (rpi - wb >= 64) {  // next window (segments longer than 64 pages)
      wb += 64 * ((rpi - wb) >> 6);
      pid = load_window(rb, wb);
      // consume here: a page-id load left in flight into the loop would
      // make the compiler wait for all vector memory operations (vmcnt(0))
      // before each later page lookup, draining the ring
      asm volatile("" ::"v"(pid));
    }
    const int pg = __builtin_amdgcn_readlane(pid, rpi - wb);
    const bool ok = (unsigned)pg < (unsigned)num_pages;
    badm |= ok ? 0u : seg_bit;
    const unsigned long long off =
        (unsigned long long)(unsigned)(ok ? pg : 0) * (unsigned)(page * kRowBytes) + (unsigned)rpo_b;
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = make_rsrc((const char*)cache + off, ok ? min(kSub, rrem) * kRowBytes : 0);
    cursor_step();
    return rf;
  };
  auto refill = [&](int pos) {
    if (rrem > 0) return refill_at(pos);
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = make_rsrc(cache, 0);
    return rf;
  };
  // sub-tile i (0 or 1) of segment k + 1 (descriptor sn), from the window
  // loaded ahead: a segment starts on a 64-token boundary, so both lie in
  // its first page
  auto refill_next = [&](int pos, const Seg& sn, int i) {
    const int pg = __builtin_amdgcn_readfirstlane(pid_next);
    const bool ok = (unsigned)pg < (unsigned)num_pages;
    badm |= (ok ? 0u : 1u) << ((k + 1) & 31);
    const long row0 = ok ? (long)pg * page + (sn.t0 % page) + kSub * i : 0;
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = make_rsrc(cache + row0 * kRow,
                      ok ? min(kSub, sn.t1 - (sn.t0 + kSub * i)) * kRowBytes : 0);
    return rf;
  };
  // past the stream, or a position that must stay unloaded: a descriptor of
  // zero bytes, so each of its loads is out of range, reads no memory and
  // writes zeros.  Issuing them keeps the count of ring loads per sub-tile
  // fixed, which the vmcnt immediates below rely on.
  auto no_refill = [&](int pos) {
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = make_rsrc(cache, 0);
    return rf;
  };

  bf16x8 qreg[kKSteps];    // absorbed query, B operand (lane = head, 8 dims per K-step half)
  auto load_q = [&](int b) {
    // The query arrives in the query-tile layout (qtile_index): each load
    // reads 1 KB contiguously.  A buffer resource on sequence b's tiles and
    // a 32-bit per-lane offset formed here: a 64-bit per-lane address would
    // be kept live across the sub-tile loop, spilled, and its reload would
    // wait for every memory operation in flight.
    const int off = (wave * kKSteps * 64 + lane_here()) * 16;
    constexpr int step = 1024;   // bytes from one K-step to the next
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q_abs + (long)b * kHeads * kRow), 0, kHeads * kRowBytes, kRsrcWord3);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8,
                                    __builtin_amdgcn_raw_buffer_load_b128(rs, off, ks * step, 0));
  };

  // the query must have landed before the sub-tile loop: a query load left in
  // flight would make the compiler wait inside the loop behind ring loads.
  // Each register is read and rewritten by an empty asm statement, so that
  // from here on its definition is that statement, not a load: the
  // compiler then has no pending load to wait for inside the loop (where
  // its vmcnt waits would also wait for the ring's loads, which it does not
  // see).
  auto consume_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qreg[ks]));
  };
  int base = 0;   // ring position of sub-tile 0 of the segment being computed
  // a pass that loads its own first two positions (the work-group's first
  // segment, or a redo): window, positions base and base + 1, then the query
  auto start_pass = [&](int b) {
    const Seg sg = seg_at(k);
    int w = load_window(sg.b, sg.t0 / page);
    asm volatile("" ::"v"(w));
    cursor_begin(k, w);
    badm &= ~(1u << (k & 31));
    const Refill r0 = refill(base);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r0, i, wave, lat16, rope_off);
    const Refill r1 = refill(base + 1);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r1, i, wave, lat16, rope_off);
    load_q(b);
    consume_q();
  };

  // the cursor of a segment whose sub-tiles 0 and 1 the previous one loaded
  auto cursor_after_prefetch = [&]() {
    cursor_begin(k, pid_next);
    cursor_step();
    cursor_step();
  };
  // work-group start: both descriptors, both page windows and the query in
  // flight together, then the first two sub-tiles (landing behind the query:
  // the first iteration waits for them itself)
  Seg cur = segs[k];
  {
    const Seg sn = segs[k + 1 < k_end ? k + 1 : k];
    asm volatile("" ::"v"(cur.b), "v"(cur.t0), "v"(cur.t1), "v"(sn.b), "v"(sn.t0));
    const int w = load_window(cur.b, cur.t0 / page);
    pid_next = load_window(sn.b, sn.t0 / page);
    load_q(cur.b);
    asm volatile("" ::"v"(w), "v"(pid_next));
    cursor_begin(k, w);
    const Refill r0 = refill(base);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r0, i, wave, lat16, rope_off);
    const Refill r1 = refill(base + 1);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r1, i, wave, lat16, rope_off);
    consume_q();
  }
  bool first_wait = true;   // iteration 0 of the first pass waits for its sub-tile

  for (;;) {   // the work-group's segments
    const bool has_next = k + 1 < k_end;
    const Seg nxt = seg_at(has_next ? k + 1 : k);
    const int nsub = (cur.t1 - cur.t0 + kSub - 1) / kSub;
    // the last two iterations load the next segment's first two sub-tiles
    // (when both segments have two or more)
    const bool pf_next = has_next && nsub >= 2 && nxt.t1 - nxt.t0 > kSub;

    f32x16 acc[16];          // acc[4 mb + n]: dims block mb of this wave x head block n
    // ---- latent accumulation operands: A[mb] = cache^T of dims block mb for
    // one K-step (two transposing reads of four tokens), B = P^T of one head
    // block (written by wave n)
    bf16x8 A[4];
    bf16x8 B[2];
    // dslot: byte distance from the bases' slot to the accumulation slot
    auto pv_read_into = [&](bf16x8(&dst)[4], int dslot, int kap) {
      static_for<0, 4>([&](auto mc) {
        constexpr int mb = decltype(mc)::value;
        const int t = tb + dslot;
        const v4bf16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf16*)((lds_char*)g_lds + xor_here<64 * mb>(t) + kLatBytes * 16 * kap));
        const v4bf16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_v4bf16*)((lds_char*)g_lds + xor_here<32 + 64 * mb>(t) + kLatBytes * (16 * kap + 2)));
        dst[mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      });
    };
    auto pv_read_at = [&](int dslot, int kap) { pv_read_into(A, dslot, kap); };
    // P^T of head block n, K-step kap (written by wave n); pb = pl + buffer
    auto p_read_at = [&](int pb, int kap, int n) {
      return lds_load<bf16x8>(pb + (2 * n + kap) * 1024);
    };
    auto pv_mfma_op = [&](const bf16x8(&op)[4], int mb, int n) {
      acc[4 * mb + n] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[mb], B[n & 1], acc[4 * mb + n], 0, 0, 0);
    };
    auto pv_mfma = [&](int mb, int n) { pv_mfma_op(A, mb, n); };
    // Softmax numerators 2^(s - m_ref) in the log2 domain (the query tiles
    // carry log2 e).  A first pass takes m_ref = 0: no subtraction at all,
    // which is exact softmax algebra as long as the numerators stay within
    // fp32 and bf16 range.  The pass tracks each head's maximum m_seen; if
    // any head of the work-group ends the segment with m_seen outside
    // [-64, 64], the segment is redone with m_ref = m_seen (numerators <= 1).
    float m_ref = 0.f;
    float l_run = 0.f;
    int mode = 0;
    for (;;) {
      // opaque to the optimiser: one copy of the sub-tile loop serves both
      // passes (a scalar: the pass decides uniform control flow)
      asm volatile("" : "+s"(mode));
      // the page windows are (re)defined here, before the loop: if the
      // register allocator parked them in scratch around the partial's
      // stores, their reload completes now, not at a page lookup inside the
      // loop (where the wait would also wait for the ring's loads)
      asm volatile("" : "+v"(pid), "+v"(pid_next));
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[x] = f32x16{};
      l_run = 0.f;
      float m_seen = -INFINITY;

      // every wave is done with the previous pass's P buffers
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();
      {
        // P buffer 1 reads as the P of sub-tile -1 in iteration 0: zero it
        // (the zeros formed here: a constant the compiler keeps for the whole
        // kernel is spilled, and its reload would wait for the ring's loads)
        uint32_t z0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
        const u32x4 z = {z0, z0, z0, z0};
        const int tl = wave * 64 + lane_here();   // formed here, not kept across the loop
        lds_store<u32x4>(kPBufOff + kPBufBytes + 16 * tl, z);
        lds_store<u32x4>(kPBufOff + kPBufBytes + 16 * (tl + kThreads), z);
      }

      // Software pipeline over sub-tiles: iteration j computes the scores of
      // sub-tile j interleaved with the latent accumulation of sub-tile j-1
      // (its P, written to LDS at the end of iteration j-1) and with the ring
      // loads of position base + j + 2; the softmax of j overlaps the last
      // quarter of j-1's accumulation.  Iteration 0 accumulates P = 0 over
      // sub-tile 0; the drain after the loop accumulates the last sub-tile.
      // Every pass starts with exactly two positions loaded ahead.
      // scalar set-up of iteration jj's ring loads (position base + jj + 2).
      // Iteration j uses the set-up formed during iteration j - 1, in the
      // shadow of its score MFMAs (between iterations the MFMAs would idle
      // through it); iteration 0's is formed here, for this pass.
      auto ring_setup = [&](int jj) {
        if (jj + 2 < nsub) return refill_at(base + jj + 2);
        if (pf_next) return refill_next(base + jj + 2, nxt, jj + 2 - nsub);
        return no_refill(base + jj + 2);
      };
      Refill rf_next = ring_setup(0);
#pragma clang loop unroll(disable)
      for (int j = 0; j < nsub; ++j) {
        const Refill rf = rf_next;
        static_assert(kInstsPerWave == 9, "vmcnt immediates below assume 9 loads per sub-tile");
        // positions base and base + 1 landed before the query did (except at
        // the work-group start); from j = 1 on, only the loads of position
        // base + j + 1 may still fly
        if (j > 0 || first_wait) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        first_wait = false;
        // this wave's P of sub-tile j-1 is in LDS before the barrier
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();  // sub-tile j landed everywhere; position base+j-2's slot is free

        const int nvalid = min(kSub, cur.t1 - (cur.t0 + j * kSub));
        const int sq_slot = (base + j) & (kSlots - 1);                    // scores tile
        const int dv = j == 0 ? 0 : (((base + j - 1) & (kSlots - 1)) - sq_slot) * kSubBytes;
        const int prd = pl + kPBufOff + ((j + 1) & 1) * kPBufBytes;   // P of sub-tile j-1
        const int pwr = pl + kPBufOff + (j & 1) * kPBufBytes;         // P of sub-tile j
        move_bases(sq_slot);

        // ---- scores for 32 tokens x 32 heads (inline asm with a VGPR
        // accumulator: with the builtin the compiler puts S in the
        // accumulation registers, which o~ already fills, and spills).
        // Back-to-back accumulation into the same registers needs no wait
        // states; the s_nop before the softmax covers MFMA-result -> VALU.
        f32x16 S;
        bf16x8 abuf[4];
        // region r < 32 runs latent K-step 8 (r & 3) + (r >> 2) (b-major),
        // regions 32..35 the RoPE K-steps
        auto ks_of = [](int r) { return r < 32 ? 8 * (r & 3) + (r >> 2) : r; };
        // the four reads of one b share one XOR-derived base, formed at the
        // first of them
        int xq = qb;
        auto a_read = [&](auto rc) {
          constexpr int r = decltype(rc)::value;
          if constexpr (r < 32) {
            if constexpr ((r & 3) == 0) xq = xor_here<32 * (r >> 2)>(qb);
            return lds_load<bf16x8>(xq + 256 * (r & 3));
          } else {
            return lds_load<bf16x8>(xor_here<(r - 32) << 5>(qrb));
          }
        };
        abuf[0] = a_read(ic<0>{});
        abuf[1] = a_read(ic<1>{});
        abuf[2] = a_read(ic<2>{});
        abuf[3] = a_read(ic<3>{});
        auto qk = [&](auto rc) {
          constexpr int r = decltype(rc)::value;
          // take this K-step's operand before its buffer slot is refilled (four
          // K-steps ahead: the LDS latency under four waves of reads)
          const bf16x8 a = abuf[r % 4];
          if constexpr (r + 4 < kKSteps) abuf[r % 4] = a_read(ic<r + 4>{});
          if constexpr (r == 0)
            score_mfma_first(S, a, qreg[ks_of(r)]);
          else
            score_mfma(S, a, qreg[ks_of(r)]);
        };

        // ---- latent accumulation of sub-tile j-1 (tile at dv from the
        // scores' slot, P at prd)
        auto p_read = [&](int kap, int n) { return p_read_at(prd, kap, n); };

        pv_read_at(dv, 0);
        B[0] = p_read(0, 0);
        // 36 regions, one score MFMA each; sched_barrier pins the interleave
        // (left alone, the scheduler clusters the builtin MFMAs away from the
        // inline-asm ones).  Regions 0..8 also issue the ring loads;
        // K-step 0 of the accumulation runs in regions 3..18, K-step 1 after
        // the score chain, beside the softmax.
        static_for<0, kKSteps>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          qk(rc);
          if constexpr (r < kInstsPerWave) ring_load(rf, r, wave, lat16, rope_off);
          // the next iteration's ring set-up (past the last iteration it
          // forms an unused descriptor: no cursor step, at most a repeated
          // mark of a bad page in the next segment)
          if constexpr (r == 12) rf_next = ring_setup(j + 1);
          if constexpr (r == 19) pv_read_at(dv, 1);
          if constexpr (r >= 3 && r < 19) {
            constexpr int idx = r - 3, n = idx >> 2, mb = idx & 3;
            if constexpr (mb == 0) B[(n + 1) & 1] = n < 3 ? p_read(0, n + 1) : p_read(1, 0);
            pv_mfma(mb, n);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        // ---- the rest of j-1's accumulation (K-step 1) with the softmax
        // numerators of sub-tile j in its shadow.  Accumulation region idx
        // runs head block idx / 4, dims block idx % 4.  The first two do not
        // read S: they cover the wait for the last score MFMA's result.
        auto tail_mfma = [&](int idx) {
          const int n = idx >> 2, mb = idx & 3;
          if (mb == 0 && n < 3) B[(n + 1) & 1] = p_read(1, n + 1);
          pv_mfma(mb, n);
        };
        tail_mfma(0);
        tail_mfma(1);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S));
        __builtin_amdgcn_sched_barrier(0);

        // Register i of lane (head, h) holds token 16 (i >> 3) + 4 (i & 3) +
        // 2 ((i >> 2) & 1) + h.  Uniform branches, both rare (a segment's
        // last, partial sub-tile; a redo pass), ahead of the block below so
        // that it stays one basic block.
        if (nvalid < kSub) {
          const int hh = lane_here() >> 5;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) + hh;
            S[i] = tok < nvalid ? S[i] : -INFINITY;
          }
        }
        if constexpr (kQLog2e) {
          // a redo pass's reference (its maxima are not used)
          if (mode != 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) S[i] -= m_ref;
          }
        }
        // 2^(s log2 e - m_ref): the subtraction above, or one fma per score
        auto num = [&](float x) {
          if constexpr (kQLog2e)
            return __builtin_amdgcn_exp2f(x);
          else
            return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -m_ref));
        };
        // Regions 2..15: the head maximum (for the pass's redo test), two
        // numerators per region from region 3, their bf16 rounding and LDS
        // write once eight are done, and the l sums over the rounded values.
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        float mx[5], l_part = 0.f;
        bf16x8 p[2];
        static_for<2, 16>([&](auto ic_) {
          constexpr int idx = decltype(ic_)::value;
          if constexpr (idx == 2) {
#pragma unroll
            for (int i = 0; i < 5; ++i) mx[i] = fmaxf(fmaxf(S[3 * i], S[3 * i + 1]), S[3 * i + 2]);
          }
          if constexpr (idx == 3) {
            float bm = fmaxf(fmaxf(mx[0], mx[1]), mx[2]);
            bm = fmaxf(fmaxf(bm, mx[3]), fmaxf(mx[4], S[15]));
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm),
                                                             __float_as_uint(bm), false, false);
            bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            if constexpr (!kQLog2e) bm *= kLog2e;
            m_seen = fmaxf(m_seen, bm);
          }
          if constexpr (idx >= 3 && idx < 11) {
            constexpr int e = 2 * (idx - 3);
            S[e] = num(S[e]);
            S[e + 1] = num(S[e + 1]);
          }
          // P of sub-tile j (B operand layout: lane = head, 8 tokens per
          // K-step half) for all four waves, and l over the rounded numbers
          // the accumulation uses (pairs of bf16 dotted with (1, 1))
          if constexpr (idx == 7 || idx == 11) {
            constexpr int kap = idx == 7 ? 0 : 1;
#pragma unroll
            for (int e = 0; e < 8; ++e) p[kap][e] = (__bf16)S[8 * kap + e];
            lds_store<bf16x8>(pwr + (2 * wave + kap) * 1024, p[kap]);
          }
          if constexpr (idx == 8 || idx == 12) {
            constexpr int kap = idx == 8 ? 0 : 1;
            static_for<0, 4>([&](auto ec) {
              constexpr int e = decltype(ec)::value;
              l_part = __builtin_amdgcn_fdot2_f32_bf16(
                  __builtin_shufflevector(p[kap], p[kap], 2 * e, 2 * e + 1), one, l_part, false);
            });
          }
          if constexpr (idx == 13) l_run += l_part;
          tail_mfma(idx);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // ---- drain: the latent accumulation of the last sub-tile.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();  // P of the last sub-tile is visible
      {
        const int dv = (((base + nsub - 1) & (kSlots - 1)) - slot_cur) * kSubBytes;
        const int prd = pl + kPBufOff + ((nsub + 1) & 1) * kPBufBytes;
        // K-step 1's cache operands go to registers of their own (A1): they
        // are read while K-step 0's MFMAs still consume A
        bf16x8 A1[4];
        pv_read_at(dv, 0);
        B[0] = p_read_at(prd, 0, 0);
        static_for<0, 16>([&](auto ic_) {
          constexpr int idx = decltype(ic_)::value, n = idx >> 2, mb = idx & 3;
          if constexpr (mb == 0)
            B[(n + 1) & 1] = n < 3 ? p_read_at(prd, 0, n + 1) : p_read_at(prd, 1, 0);
          if constexpr (idx == 4) pv_read_into(A1, dv, 1);
          pv_mfma(mb, n);
          __builtin_amdgcn_sched_barrier(0);
        });
        static_for<0, 16>([&](auto ic_) {
          constexpr int idx = decltype(ic_)::value, n = idx >> 2, mb = idx & 3;
          if constexpr (mb == 0 && n < 3) B[(n + 1) & 1] = p_read_at(prd, 1, n + 1);
          pv_mfma_op(A1, mb, n);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // A head maximum outside [-64, 64] anywhere in the work-group: redo
      // the segment with the exact maxima seen in this pass (rare).  Each
      // wave votes for its 32 heads (m_seen is per head, so the OR over its
      // lanes) in P buffer nsub & 1, which no wave reads after the drain's
      // barrier (its last reader was iteration nsub - 1).  The redo starts at
      // the ring position after this pass, behind the loads in flight there
      // (same slots, issued earlier by the same wave, so they land earlier).
      if (mode == 0) {
        const int pv = kPBufOff + (nsub & 1) * kPBufBytes;
        const bool mine = __builtin_amdgcn_ballot_w64(!(fabsf(m_seen) <= kLazy)) != 0;
        if (lane_here() == 0) lds_store<uint32_t>(pv + 4 * wave, mine ? 1u : 0u);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_barrier();
        const u32x4 votes = lds_load<u32x4>(pv);
        // the same words in every lane: a uniform decision
        if (__builtin_amdgcn_readfirstlane(votes[0] | votes[1] | votes[2] | votes[3]) != 0) {
          m_ref = m_seen;
          mode = 1;
          base += nsub;
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          start_pass(cur.b);
          continue;
        }
      }
      break;
    }
    base += nsub;

    // The query registers are free from here on: the next segment's query
    // loads now, under the partial's write.  (Issued here rather than in the
    // drain: there, on the path that leaves the pass loop, the compiler's
    // wait analysis would carry the loads as outstanding into the next
    // pass's sub-tile loop and wait for them at every score step - waits
    // that would also drain the ring.)
    if (has_next) load_q(nxt.b);

    // the window of the segment after the next, issued before the partial's
    // stores so that waiting for it does not wait for the stores
    int pid_n2 = 0;
    if (k + 2 < k_end) {
      const Seg s2 = seg_at(k + 2);
      pid_n2 = load_window(s2.b, s2.t0 / page);
    }

    // ---- unnormalised partial (m, l, o~): o~ rounded to bf16, in register
    // order (16-byte piece 2x + e of a lane holds elements 8e .. 8e + 7 of
    // accumulator x); merged later
    {
      const int ln = lane_here();
      uint4* dst = (uint4*)(part_o + (long)k * kHeads * kDc) + (wave * 64 + ln);
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w[j] = __builtin_bit_cast(
                uint32_t, bf16x2{(__bf16)acc[x][8 * e + 2 * j], (__bf16)acc[x][8 * e + 2 * j + 1]});
          dst[(x * 2 + e) * kThreads] = uint4{w[0], w[1], w[2], w[3]};
          // one accumulator at a time: the next query is arriving in the
          // VGPRs, and reading all accumulators ahead would not fit beside it
          if (e == 1) __builtin_amdgcn_sched_barrier(0);
        }
      // l over all 32 tokens of a sub-tile: lanes (m32, 0) and (m32, 1) hold
      // halves of head m32's sum
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                       __float_as_uint(l_run), false, false);
      const float l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const bool bad = (badm >> (k & 31)) & 1u;
      badm &= ~(1u << (k & 31));
      if (ln < 32) {
        float2* ml = (float2*)(part_ml + ((long)k * kHeads + wave * 32 + ln) * 2);
        *ml = float2{m_ref * kLn2, bad ? __builtin_nanf("") : l_tot};
      }
    }
    if (!has_next) break;
    ++k;
    cur = nxt;
    if (!pf_next) {
      // a short segment on either side: the next one loads its own start
      consume_q();
      asm volatile("" ::"v"(pid_n2));
      pid_next = pid_n2;
      start_pass(cur.b);
      continue;
    }
    consume_q();
    asm volatile("" ::"v"(pid_n2));
    cursor_after_prefetch();   // from pid_next: the window of segment k
    pid_next = pid_n2;
  }
}

// Rows [B][128][576] -> query tiles (qtile_index), values unchanged: one
// 16-byte piece (eight consecutive numbers of one row, which stay
// consecutive) per thread.
__global__ __launch_bounds__(256) void qtile_pack_kernel(const uint4* __restrict__ rows, long n,
                                                         uint4* __restrict__ tiles) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const long r = p / (kRow / 8);                  // row = m * 128 + head
  const int d = 8 * (int)(p - r * (kRow / 8));
  tiles[qtile_index(r / kHeads, (int)(r % kHeads), d) / 8] = rows[p];
}

// ---------------------------------------------------------------------------
// merge of the register-order partials: one work-group per (sequence, head
// block of 32).  o~ = sum_s e^(m_s - M) o~_s / sum_s e^(m_s - M) l_s.
// ---------------------------------------------------------------------------
constexpr int kCombSegs = 64;   // segments weighed per pass

__global__ __launch_bounds__(512) void combine_v2_kernel(PlanPtrs plan,
                                                         const __bf16* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         __bf16* __restrict__ lat_out) {
  __shared__ float w[kCombSegs][32];
  __shared__ float2 s_ml[kCombSegs][32];
  __shared__ float s_M[32], s_inv[32];
  __shared__ __bf16 stage[32][kDc + 8];
  __shared__ f32x4 s_acc[16][256];   // the odd-segment half's sums
  const int b = blockIdx.x, n = blockIdx.y, t = threadIdx.x;
  const int half = t >> 8, tt = t & 255;   // tt: the accumulator slot, as below
  const int cnt = plan.seq_seg_count[b];
  const int k0 = plan.seq_seg_start[b];
  __bf16* out = lat_out + ((long)b * kHeads + n * 32) * kDc;
  if (cnt == 0) {
    for (int e = t; e < 32 * kDc; e += 512) out[e] = (__bf16)__builtin_nanf("");
    return;
  }
  // thread t takes lane tt & 63 of the attention kernel's wave wo = tt >> 6,
  // whose accumulators x = 4 mb + n hold latent dims [128 wo, 128 wo + 128);
  // the two halves of the work-group sum the even and the odd segments, four
  // segments' loads in flight per half at once
  constexpr int kU = 4;
  uint4 v[kU][8];   // [u][2 mb + e]: elements 8e .. 8e + 7 of accumulator 4 mb + n
  auto load_round = [&](int c0, int s0, int nc) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + 2 * u >= nc) break;
      const uint4* src = (const uint4*)(part_o + (long)(k0 + c0 + s0 + 2 * u) * kHeads * kDc) + tt;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 2; ++e) v[u][2 * mb + e] = src[((4 * mb + n) * 2 + e) * kThreads];
    }
  };
  // the first round's partials go out before the softmax statistics, which
  // they do not depend on: their memory round trip overlaps that of (m, l)
  load_round(0, half, min(kCombSegs, cnt));
  // (m, l) of every segment of the head group: one parallel load into LDS
  // when they fit (else read in the loops below)
  const bool in_lds = cnt <= kCombSegs;
  if (in_lds)
    for (int e = t; e < cnt * 32; e += 512)
      s_ml[e >> 5][e & 31] =
          *(const float2*)(part_ml + ((long)(k0 + (e >> 5)) * kHeads + n * 32 + (e & 31)) * 2);
  __syncthreads();
  auto ml_of = [&](int s, int hh) -> float2 {
    if (in_lds) return s_ml[s][hh];
    return *(const float2*)(part_ml + ((long)(k0 + s) * kHeads + n * 32 + hh) * 2);
  };
  // per-head max and normaliser
  if (t < 32) {
    float M = -INFINITY;
    for (int s = 0; s < cnt; ++s) M = fmaxf(M, ml_of(s, t).x);
    float L = 0.f;
    for (int s = 0; s < cnt; ++s) {
      const float2 ml = ml_of(s, t);
      L += ml.y * __expf(ml.x - M);
    }
    s_M[t] = M;
    s_inv[t] = 1.f / L;
  }
  __syncthreads();
  const int lane = tt & 63, wo = tt >> 6;
  const int hd_l = lane & 31;
  f32x4 acc[16];   // [4 mb + a]
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = f32x4{};
  for (int c0 = 0; c0 < cnt; c0 += kCombSegs) {
    const int nc = min(kCombSegs, cnt - c0);
    __syncthreads();
    for (int e = t; e < nc * 32; e += 512) {
      const int s = e >> 5, hh = e & 31;
      w[s][hh] = __expf(ml_of(c0 + s, hh).x - s_M[hh]) * s_inv[hh];
    }
    __syncthreads();
    // each half sums its segments in order
    for (int s0 = half; s0 < nc; s0 += 2 * kU) {
      if (c0 > 0 || s0 != half) load_round(c0, s0, nc);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (s0 + 2 * u >= nc) break;
        const float ws = w[s0 + 2 * u][hd_l];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          acc[2 * r] += ws * f32x4{__uint_as_float(v[u][r].x << 16),
                                   __uint_as_float(v[u][r].x & 0xffff0000u),
                                   __uint_as_float(v[u][r].y << 16),
                                   __uint_as_float(v[u][r].y & 0xffff0000u)};
          acc[2 * r + 1] += ws * f32x4{__uint_as_float(v[u][r].z << 16),
                                       __uint_as_float(v[u][r].z & 0xffff0000u),
                                       __uint_as_float(v[u][r].w << 16),
                                       __uint_as_float(v[u][r].w & 0xffff0000u)};
        }
      }
    }
  }
  if (half == 1)
#pragma unroll
    for (int r = 0; r < 16; ++r) s_acc[r][tt] = acc[r];
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += s_acc[r][tt];
    // register order -> [head][dim]: element i = 4a + c of accumulator
    // (mb, n) at lane (m32, hf) is head 32n + m32, dim 128 wo + 32 mb + 8a + 4 hf + c
    const int hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          stage[hd_l][128 * wo + 32 * mb + 8 * a + 4 * hf + c] = (__bf16)acc[4 * mb + a][c];
  }
  __syncthreads();
  for (int e = t; e < 32 * (kDc / 8); e += 512) {
    const int hh = e / (kDc / 8), c8 = e % (kDc / 8);
    *(uint4*)(out + (long)hh * kDc + 8 * c8) = *(const uint4*)(&stage[hh][8 * c8]);
  }
}

// ---------------------------------------------------------------------------
// the same merge for small batches: one work-group of kRunWaves waves per
// (sequence, head block n of 32, latent run of 32 dims).  Accumulator
// x = 4 mb + n of the attention kernel's wave wo holds, in element 4a + c at
// lane (m32, hf), head 32n + m32 and dim 128 wo + 32 mb + 8a + 4 hf + c; the
// work-group z = 4 wo + mb takes all of accumulator (mb, n): dims
// 128 wo + 32 mb .. + 31, one contiguous run.  Sixteen times the work-groups of
// combine_v2_kernel, so that a few sequences with many segments each still
// spread over the GPU; within a work-group wave q sums the segments
// s = q (mod kRunWaves), the first loads are issued before the softmax
// statistics are formed, and the waves' sums are added at the end in a fixed
// order.
// ---------------------------------------------------------------------------
constexpr int kRunWaves = 8;   // waves per merge work-group, each a share of the segments
constexpr int kRunSegs = 264;   // (m, l) kept in LDS: every automatic plan (<= CUs + 1 segments)

__global__ __launch_bounds__(64 * kRunWaves) void combine_v2_runs_kernel(PlanPtrs plan,
                                                         const __bf16* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         __bf16* __restrict__ lat_out) {
  __shared__ float2 s_ml[kRunSegs][32];   // (m, l), then the segment weights in .x
  __shared__ float s_M[32], s_inv[32];
  __shared__ f32x4 s_acc[kRunWaves - 1][4][64];   // the sums of waves 1 ..
  __shared__ __bf16 stage[32][32 + 8];
  const int b = blockIdx.x, n = blockIdx.y, wo = blockIdx.z >> 2, mz = blockIdx.z & 3;
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;
  const int cnt = plan.seq_seg_count[b];
  const int k0 = plan.seq_seg_start[b];
  __bf16* out = lat_out + ((long)b * kHeads + n * 32) * kDc + 128 * wo + 32 * mz;
  if (cnt == 0 || cnt > kRunSegs) {
    // no valid segment: NaN.  (More segments than kRunSegs come only from a
    // forced split count beyond the work-group budget; the host sends those
    // to combine_v2_kernel.)
    for (int e = tid; e < 32 * 32; e += 64 * kRunWaves)
      out[(e >> 5) * kDc + (e & 31)] = (__bf16)__builtin_nanf("");
    return;
  }
  const int hd_l = lane & 31;
  // this wave's segments s = q, q + kRunWaves, ...: the first kU in flight now
  constexpr int kU = 8;
  uint4 v[kU][2];   // [u][e]: elements 8e .. 8e + 7 of accumulator 4 mz + n
  auto issue = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int su = min(s0 + kRunWaves * u, cnt - 1);   // past the end: re-read, weight 0
      const uint4* src =
          (const uint4*)(part_o + (long)(k0 + su) * kHeads * kDc) + wo * 64 + lane;
#pragma unroll
      for (int e = 0; e < 2; ++e) v[u][e] = src[((4 * mz + n) * 2 + e) * kThreads];
    }
  };
  issue(q);
  for (int e = tid; e < cnt * 32; e += 64 * kRunWaves)
    s_ml[e >> 5][e & 31] =
        *(const float2*)(part_ml + ((long)(k0 + (e >> 5)) * kHeads + n * 32 + (e & 31)) * 2);
  __syncthreads();
  // per-head max and normaliser: lane pair (hd, hd + 32) of wave 0 splits the
  // segments by parity
  if (q == 0) {
    const int h2 = lane >> 5;
    float M = -INFINITY;
    for (int s = h2; s < cnt; s += 2) M = fmaxf(M, s_ml[s][hd_l].x);
    M = fmaxf(M, __shfl_xor(M, 32));
    float L = 0.f;
    for (int s = h2; s < cnt; s += 2) L += s_ml[s][hd_l].y * __expf(s_ml[s][hd_l].x - M);
    L += __shfl_xor(L, 32);
    if (h2 == 0) {
      s_M[hd_l] = M;
      s_inv[hd_l] = 1.f / L;
    }
  }
  __syncthreads();
  for (int e = tid; e < cnt * 32; e += 64 * kRunWaves) {
    const int s = e >> 5, hh = e & 31;
    s_ml[s][hh].x = __expf(s_ml[s][hh].x - s_M[hh]) * s_inv[hh];
  }
  __syncthreads();
  f32x4 acc[4];   // [a]
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = f32x4{};
  for (int s0 = q; s0 < cnt; s0 += kRunWaves * kU) {
    if (s0 != q) issue(s0);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int su = s0 + kRunWaves * u;
      if (su >= cnt) continue;
      const float ws = s_ml[su][hd_l].x;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        acc[2 * e] += ws * f32x4{__uint_as_float(v[u][e].x << 16),
                                 __uint_as_float(v[u][e].x & 0xffff0000u),
                                 __uint_as_float(v[u][e].y << 16),
                                 __uint_as_float(v[u][e].y & 0xffff0000u)};
        acc[2 * e + 1] += ws * f32x4{__uint_as_float(v[u][e].z << 16),
                                     __uint_as_float(v[u][e].z & 0xffff0000u),
                                     __uint_as_float(v[u][e].w << 16),
                                     __uint_as_float(v[u][e].w & 0xffff0000u)};
      }
    }
  }
  if (q > 0)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) s_acc[q - 1][mb][lane] = acc[mb];
  __syncthreads();
  if (q == 0) {
    // the waves' sums added in a fixed order
#pragma unroll
    for (int w = 0; w < kRunWaves - 1; ++w)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] += s_acc[w][mb][lane];
    // element c of acc[a] at lane (m32, hf): head 32n + m32, dim
    // 8 a + 4 hf + c of this work-group's run
    const int hf = lane >> 5;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) stage[hd_l][8 * a + 4 * hf + c] = (__bf16)acc[a][c];
  }
  __syncthreads();
  if (tid < 128) {
    const int hh = tid >> 2, c8 = tid & 3;
    *(uint4*)(out + (long)hh * kDc + 8 * c8) = *(const uint4*)(&stage[hh][8 * c8]);
  }
}

}  // namespace

hipError_t attn_decode_v2(const Geo& g, const void* q_tiles, bool q_log2e, const void* cache,
                          int num_pages, const int32_t* page_table, int max_pages,
                          const PlanPtrs& plan, int n_wg_launch, void* part_o, float* part_ml,
                          hipStream_t s) {
  if (n_wg_launch <= 0) return hipSuccess;
  if (q_log2e)
    hipLaunchKernelGGL(attn_v2_kernel<true>, dim3(n_wg_launch), dim3(kThreads), 0, s,
                       (const __bf16*)q_tiles, (const __bf16*)cache, num_pages, page_table,
                       max_pages, g.page, (const int*)plan.counts, (const int*)plan.wg_seg_start,
                       (const Seg*)plan.segs, (__bf16*)part_o, part_ml);
  else
    hipLaunchKernelGGL(attn_v2_kernel<false>, dim3(n_wg_launch), dim3(kThreads), 0, s,
                       (const __bf16*)q_tiles, (const __bf16*)cache, num_pages, page_table,
                       max_pages, g.page, (const int*)plan.counts, (const int*)plan.wg_seg_start,
                       (const Seg*)plan.segs, (__bf16*)part_o, part_ml);
  return hipGetLastError();
}

hipError_t pack_query_tiles(const void* rows, int B, void* tiles, hipStream_t s) {
  const long n = (long)B * kHeads * (kRow / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(qtile_pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const uint4*)rows, n, (uint4*)tiles);
  return hipGetLastError();
}

hipError_t combine_decode_v2(const PlanPtrs& plan, int B, int num_splits, const void* part_o,
                             const float* part_ml, void* lat_out, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  // 4 B work-groups of 256 threads fill the GPU for batches from 32 up; below
  // that, 64 B two-wave work-groups, as long as a sequence's segments fit
  // their LDS table (an automatic plan makes at most work-groups + 1; a forced
  // one, num_splits)
  const int max_per_seq = num_splits > 0 ? num_splits : plan_dims(B, 0).max_wg + 1;
  if (B >= 32 || max_per_seq > kRunSegs)
    hipLaunchKernelGGL(combine_v2_kernel, dim3(B, kHeads / 32), dim3(512), 0, s, plan,
                       (const __bf16*)part_o, part_ml, (__bf16*)lat_out);
  else
    hipLaunchKernelGGL(combine_v2_runs_kernel, dim3(B, kHeads / 32, 4 * kWaves),
                       dim3(64 * kRunWaves), 0, s, plan, (const __bf16*)part_o, part_ml, (__bf16*)lat_out);
  return hipGetLastError();
}

}  // namespace mla
