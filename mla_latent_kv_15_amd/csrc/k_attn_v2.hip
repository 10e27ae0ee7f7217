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
//  * 32-token sub-tiles stream through a four-slot LDS ring with 16-byte
//    direct-to-LDS buffer loads, two sub-tiles in flight while the scores of
//    sub-tile j and the accumulation of sub-tile j-1 run.  A slot holds the
//    32 latent parts (1024 B each) and then the 32 RoPE parts (128 B each);
//    16-byte pieces are XOR-permuted per row so that every LDS read pattern
//    below is free of bank conflicts, and each ring load covers exactly one
//    row's latent part (or the RoPE parts of eight rows), which keeps its
//    address arithmetic to one or two instructions.
//  * scores: S^T[token][head] = C[token][dims] . Q~^T[dims][head] with
//    v_mfma_f32_32x32x16_bf16 (A = cache rows from LDS, B = Q~), 36 K-steps.
//  * softmax numerators in the log2 domain against a per-segment reference:
//    the max of the segment's first 32 scores.  Later scores may exceed it by
//    up to 64 (P <= 2^64, harmless in fp32/bf16), so the 256-register
//    accumulator is never rescaled - VALU work on it would push the kernel
//    out of its 512-register budget.  If any score in the work-group exceeds
//    the reference by more than 64, the segment is redone once with the exact
//    maximum, which the first pass tracks (correct for any input, essentially
//    never taken).
//  * latent accumulation: o~^T[dims][head] += C^T[dims][tokens] . P^T.  Each
//    lane reads 4 dims of 8 tokens (ds_read_b64) and transposes them with
//    v_perm_b32 into the A operand; P^T comes from LDS.
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
constexpr float kLazy = 64.0f;        // allowed score excess over the reference (log2 units)
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer resource, gfx9 family

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

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
// the resource's base go to LDS slot `slot`.  Rows at or past nvalid
// (rmax = nvalid - 1) re-read row rmax: their scores are masked to zero
// weight and the data stays finite, so 0 * row never turns into NaN.  Wave w
// moves rows [8w, 8w+8): loads 0..7 the latent part of one row each, load 8
// the RoPE parts of all eight.  Every wave issues exactly kInstsPerWave loads
// per sub-tile whatever nvalid is; the ring's vmcnt bookkeeping relies on it.
//
// The loads are MUBUF (buffer_load ... lds) rather than global_load_lds: the
// compiler treats an outstanding FLAT-encoded LDS load as an LDS access of
// unknown order and then waits for every LDS read with lgkmcnt(0), which
// would serialise the operand prefetch of the compute loop.
struct Refill {
  __amdgpu_buffer_rsrc_t rs;
  int slot;   // LDS byte offset of the ring slot
  int rmax;
};

__device__ inline void ring_load(const Refill& rf, int i, int wave, int lane) {
  int w = wave, l = lane;
  asm volatile("" : "+s"(w), "+v"(l));  // recompute per call: no live per-load state
  if (i < 8) {
    const int r = 8 * w + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rf.rs, (lds_void*)((lds_char*)g_lds + rf.slot + r * kLatBytes), 16,
        (l << 4) ^ ((r & 15) << 4), min(r, rf.rmax) * kRowBytes, 0, 0);
  } else {
    const int r = 8 * w + (l >> 3);   // this lane's row; piece l & 7 of its RoPE part
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rf.rs, (lds_void*)((lds_char*)g_lds + rf.slot + kRopeOff + 8 * w * kRopeBytes), 16,
        min(r, rf.rmax) * kRowBytes + kLatBytes + (((l & 7) ^ swz_rope(r)) << 4), 0, 0, 0);
  }
}

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
  const int head = wave * 32 + m32;

  // Per-lane LDS byte offsets within a ring slot.
  // scores, latent K-step ks: row m32, piece 2ks + h at position
  // (2ks + h) ^ (m32 & 15)  ->  (qa ^ ((ks & 7) << 5)) + 256 (ks >> 3)
  const int qa = m32 * kLatBytes + ((h ^ (m32 & 15)) << 4);
  // scores, RoPE K-step 32 + r: row m32, RoPE piece 2r + h -> qra ^ (r << 5)
  const int qra = kRopeOff + m32 * kRopeBytes + ((h ^ swz_rope(m32)) << 4);
  // accumulation, element e = 4a + c of the 8 tokens of lane (m32, h): token
  // row R = 16 kap + 8a + 4h + c, dims 4 m32 .. 4 m32 + 3 of this wave's 128,
  // i.e. latent piece 16w + (m32 >> 1), half m32 & 1:
  // (pa ^ ((8a + c) << 4)) + (16 kap + 8a + c) * 1024
  const int pa = 4 * h * kLatBytes + 256 * wave + (((m32 >> 1) ^ (4 * h)) << 4) + 8 * (m32 & 1);
  auto slot_off = [](int pos) { return kRingOff + (pos & (kSlots - 1)) * kSubBytes; };

  // Page ids, 64 pages per window: lane i holds the id of page w0 + i of
  // sequence b (-1 past the table row).  A vector register instead of scalar
  // loads: an outstanding scalar load would force a full LDS wait
  // (lgkmcnt(0)) at every use of an LDS read in the loop below.
  auto load_window = [&](int b, int w0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int p = w0 + ln;
    return p < max_pages ? page_table[(long)b * max_pages + p] : -1;
  };

  // ---- ring refill cursor.  The work-group's sub-tiles form one stream
  // (segment after segment); ring position pos holds a stream sub-tile in
  // slot pos mod 4.  Each computing iteration consumes one position and loads
  // the one two ahead, so near a segment's end the cursor walks into the
  // next segment and that segment's first sub-tiles arrive while this one is
  // still computed.  Cursor: segment rk (sequence rb), next token rt, end rt1,
  // rn sub-tiles left, at offset rpo of page rpi, page window wb / pid.
  int rk = k_begin, rb = 0, rt = 0, rt1 = 0, rn = 0, rpi = 0, rpo = 0, wb = 0, pid = 0;
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
    rk = kk;
    rb = sg.b;
    rt = sg.t0;
    rt1 = sg.t1;
    rn = (sg.t1 - sg.t0 + kSub - 1) / kSub;
    wb = sg.t0 / page;
    rpi = wb;
    rpo = sg.t0 - wb * page;
    pid = w;
  };
  // the cursor's next sub-tile, for ring position pos (sub-tiles never
  // straddle a page: page is a multiple of 64 and segments start on 64-token
  // boundaries or at 0)
  auto refill = [&](int pos) {
    Refill rf;
    rf.slot = slot_off(pos);
    if (rn > 0) {
      if (rpi - wb >= 64) {  // next window (segments longer than 64 pages)
        wb += 64 * ((rpi - wb) >> 6);
        pid = load_window(rb, wb);
        // consume here: a page-id load left in flight into the loop would
        // make the compiler wait for all vector memory operations (vmcnt(0))
        // before each later page lookup, draining the ring
        asm volatile("" ::"v"(pid));
      }
      const int pg = __builtin_amdgcn_readlane(pid, rpi - wb);
      const bool ok = pg >= 0 && pg < num_pages;
      badm |= (ok ? 0u : 1u) << (rk & 31);
      const long row0 = ok ? (long)pg * page + rpo : 0;
      rf.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(cache + row0 * kRow), 0, kSubBytes,
                                                kRsrcWord3);
      rf.rmax = ok ? min(kSub, rt1 - rt) - 1 : 0;
      --rn;
      rt += kSub;
      rpo += kSub;
      if (rpo == page) {
        rpo = 0;
        ++rpi;
      }
    } else {
      rf.rs = __builtin_amdgcn_make_buffer_rsrc((void*)cache, 0, 0, kRsrcWord3);
      rf.rmax = 0;
    }
    return rf;
  };
  // past the stream, or a position that must stay unloaded: a resource of zero
  // bytes, so each of its loads is out of range and moves no data.  Issuing
  // them keeps the count of ring loads per sub-tile fixed, which the vmcnt
  // immediates below rely on.
  // sub-tile i (0 or 1) of segment k + 1 (descriptor sn), from the window
  // loaded ahead: a segment starts on a 64-token boundary, so both lie in
  // its first page
  auto refill_next = [&](int pos, const Seg& sn, int i) {
    const int pg = __builtin_amdgcn_readfirstlane(pid_next);
    const bool ok = pg >= 0 && pg < num_pages;
    badm |= (ok ? 0u : 1u) << ((k + 1) & 31);
    const long row0 = ok ? (long)pg * page + (sn.t0 % page) + kSub * i : 0;
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(cache + row0 * kRow), 0, kSubBytes,
                                              kRsrcWord3);
    rf.rmax = ok ? min(kSub, sn.t1 - (sn.t0 + kSub * i)) - 1 : 0;
    return rf;
  };
  auto no_refill = [&](int pos) {
    Refill rf;
    rf.slot = slot_off(pos);
    rf.rs = __builtin_amdgcn_make_buffer_rsrc((void*)cache, 0, 0, kRsrcWord3);
    rf.rmax = 0;
    return rf;
  };

  bf16x8 qreg[kKSteps];    // absorbed query, B operand (lane = head, 8 dims per K-step half)
  auto load_q = [&](int b) {
    // The query arrives in the query-tile layout (qtile_index): each load
    // reads 1 KB contiguously (in rows, 16 B from each of 64 rows 1152 B
    // apart, the loads took several microseconds per segment).  A buffer
    // resource on sequence b's tiles and a 32-bit per-lane offset formed
    // here: a 64-bit per-lane address would be kept live across the sub-tile
    // loop, spilled, and its reload would wait for every memory operation in
    // flight.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int off = (wave * kKSteps * 64 + ln) * 16;
    constexpr int step = 1024;   // bytes from one K-step to the next
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(q_abs + (long)b * kHeads * kRow), 0, kHeads * kRowBytes, kRsrcWord3);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8,
                                    __builtin_amdgcn_raw_buffer_load_b128(rs, off, ks * step, 0));
  };


  // the query must have landed before the sub-tile loop: a query load left in
  // flight would make the compiler wait inside the loop behind ring loads
  auto consume_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" ::"v"(qreg[ks]));
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
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r0, i, wave, lane);
    const Refill r1 = refill(base + 1);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r1, i, wave, lane);
    load_q(b);
    consume_q();
  };

  // the cursor of a segment whose sub-tiles 0 and 1 the previous one loaded
  auto cursor_after_prefetch = [&]() {
    cursor_begin(k, pid_next);
    rn -= 2;
    rt += 2 * kSub;
    rpo += 2 * kSub;
    if (rpo == page) {
      rpo = 0;
      ++rpi;
    }
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
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r0, i, wave, lane);
    const Refill r1 = refill(base + 1);
#pragma unroll
    for (int i = 0; i < kInstsPerWave; ++i) ring_load(r1, i, wave, lane);
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
    // ---- latent accumulation, K-step kap (16 tokens) of the tile at LDS
    // offset pvb - pa: 8 x ds_read_b64 -> 16 v_perm_b32 -> A operands of the
    // 4 dims blocks; P^T of head block n from the P buffer at prd
    u32x2 raw[8];
    bf16x8 A[4];
    bf16x8 B[2];
    auto pv_read_at = [&](int pvb, int kap) {
      static_for<0, 8>([&](auto ec) {
        constexpr int e = decltype(ec)::value, a = e >> 2, c = e & 3;
        raw[e] = lds_load<u32x2>(xor_here<(8 * a + c) << 4>(pvb) + (16 * kap + 8 * a + c) * kLatBytes);
      });
    };
    auto pv_build = [&]() {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        u32x4 t;
#pragma unroll
        for (int f = 0; f < 4; ++f)
          t[f] = __builtin_amdgcn_perm(raw[2 * f + 1][mb >> 1], raw[2 * f][mb >> 1],
                                       (mb & 1) ? 0x07060302u : 0x05040100u);
        A[mb] = __builtin_bit_cast(bf16x8, t);
      }
    };
    // P^T of head block n, K-step kap (written by wave n)
    auto p_read_at = [&](int prd, int kap, int n) {
      int l = lane;
      asm volatile("" : "+v"(l));
      return lds_load<bf16x8>(prd + (2 * n + kap) * 1024 + 16 * l);
    };
    auto pv_mfma = [&](int mb, int n) {
      acc[4 * mb + n] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[mb], B[n & 1], acc[4 * mb + n], 0, 0, 0);
    };
    float m_ref = -INFINITY; // exponent reference (log2 units), fixed within a pass
    float l_run = 0.f;
    // pass 0: reference = max of the first 32 tokens; every sub-tile's max is
    // tracked, so after a pass-0 overflow the exact segment max is known and
    // pass 1 redoes the segment with it as the reference
    int mode = 0;
    for (;;) {
      // opaque to the optimiser: one copy of the sub-tile loop serves both
      // passes (a scalar: the pass decides uniform control flow)
      asm volatile("" : "+s"(mode));
#pragma unroll
      for (int x = 0; x < 16; ++x) acc[x] = f32x16{};
      l_run = 0.f;
      float m_seen = -INFINITY;
      bool over = false;

      // every wave is done with the previous pass's P buffers
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();
      {
        // P buffer 1 reads as the P of sub-tile -1 in iteration 0: zero it
        const u32x4 z = {};
        int ln = lane;
        asm volatile("" : "+v"(ln));   // the address is formed here, not kept across the loop
        const int tl = wave * 64 + ln;
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
#pragma clang loop unroll(disable)
      for (int j = 0; j < nsub; ++j) {
        // scalar set-up of the ring loads (issued below), ahead of the waits
        Refill rf;
        if (j + 2 < nsub)
          rf = refill(base + j + 2);
        else if (pf_next)
          rf = refill_next(base + j + 2, nxt, j + 2 - nsub);
        else
          rf = no_refill(base + j + 2);
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
        const int sq = slot_off(base + j);                       // scores tile
        const int sv = j == 0 ? sq : slot_off(base + j - 1);     // accumulation tile
        const int prd = kPBufOff + ((j + 1) & 1) * kPBufBytes;   // P of sub-tile j-1
        const int pwr = kPBufOff + (j & 1) * kPBufBytes;         // P of sub-tile j

        // ---- scores for 32 tokens x 32 heads (inline asm with a VGPR
        // accumulator: with the builtin the compiler puts S in the
        // accumulation registers, which o~ already fills, and spills).
        // Back-to-back accumulation into the same registers needs no wait
        // states; the s_nop before the softmax covers MFMA-result -> VALU.
        f32x16 S;
        bf16x8 abuf[4];
        const int qab = sq + qa, qrb = sq + qra;
        auto a_read = [&](auto ksc) {
          constexpr int ks = decltype(ksc)::value;
          if constexpr (ks < 32)
            return lds_load<bf16x8>(xor_here<(ks & 7) << 5>(qab) + 256 * (ks >> 3));
          else
            return lds_load<bf16x8>(xor_here<(ks - 32) << 5>(qrb));
        };
        abuf[0] = a_read(ic<0>{});
        abuf[1] = a_read(ic<1>{});
        abuf[2] = a_read(ic<2>{});
        abuf[3] = a_read(ic<3>{});
        auto qk = [&](auto ksc) {
          constexpr int ks = decltype(ksc)::value;
          // take this K-step's operand before its buffer slot is refilled (four
          // K-steps ahead: the LDS latency under four waves of reads)
          const bf16x8 a = abuf[ks % 4];
          if constexpr (ks + 4 < kKSteps) abuf[ks % 4] = a_read(ic<ks + 4>{});
          if constexpr (ks == 0)
            score_mfma_first(S, a, qreg[ks]);
          else
            score_mfma(S, a, qreg[ks]);
        };

        // ---- latent accumulation of sub-tile j-1 (tile at sv, P at prd)
        const int pvb = sv + pa;
        auto pv_read = [&](int kap) { pv_read_at(pvb, kap); };
        auto p_read = [&](int kap, int n) { return p_read_at(prd, kap, n); };

        pv_read(0);
        B[0] = p_read(0, 0);
        // 36 regions, one score MFMA each; sched_barrier pins the interleave
        // (left alone, the scheduler clusters the builtin MFMAs away from the
        // inline-asm ones).  Regions 0..8 also issue the ring loads;
        // K-step 0 of the accumulation runs in regions 3..18, K-step 1 after
        // the score chain, beside the softmax.
        static_for<0, kKSteps>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          qk(rc);
          if constexpr (r < kInstsPerWave) ring_load(rf, r, wave, lane);
          if constexpr (r == 2 || r == 19) pv_build();
          if constexpr (r == 14) pv_read(1);
          if constexpr (r >= 3 && r < 19) {
            constexpr int idx = r - 3, n = idx >> 2, mb = idx & 3;
            if constexpr (mb == 0) B[(n + 1) & 1] = n < 3 ? p_read(0, n + 1) : p_read(1, 0);
            pv_mfma(mb, n);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(S));

        // ---- softmax numerators of sub-tile j (log2 domain), lane = head, 16
        // of the 32 tokens; overlaps the rest of j-1's accumulation
        if (nvalid < kSub) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = 8 * (i >> 2) + 4 * h + (i & 3);
            S[i] = tok < nvalid ? S[i] : -INFINITY;
          }
        }
        float mx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) mx[i] = fmaxf(S[i], S[i + 8]);
#pragma unroll
        for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], mx[i + 4]);
        float bm = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm),
                                                           false, false);
          bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * kLog2e;
        }
        m_seen = fmaxf(m_seen, bm);
        // pass 0 takes its reference from the first sub-tile (m_ref is -inf
        // until then); the redo pass starts with the exact maximum
        m_ref = (m_ref == -INFINITY) ? bm : m_ref;
        over |= bm > m_ref + kLazy;
        // the numerators beside the first eight accumulation MFMAs, their
        // LDS write beside the last eight (which hides its latency before
        // the next barrier)
#pragma unroll
        for (int idx = 0; idx < 8; ++idx) {
          const int n = idx >> 2, mb = idx & 3;
          if (mb == 0) B[(n + 1) & 1] = p_read(1, n + 1);
          pv_mfma(mb, n);
          S[2 * idx] = __builtin_amdgcn_exp2f(fmaf(S[2 * idx], kLog2e, -m_ref));
          S[2 * idx + 1] = __builtin_amdgcn_exp2f(fmaf(S[2 * idx + 1], kLog2e, -m_ref));
        }
        // P of sub-tile j (B operand layout: lane = head, 8 tokens per K-step
        // half) for all four waves.  The last sub-tile of a first pass
        // carries the wave's redo vote in the sign bit of lane 0's first
        // number: the numerators are never negative, and a redo discards
        // everything they feed.
        const bool vote = mode == 0 && j == nsub - 1 && over;
#pragma unroll
        for (int kap = 0; kap < 2; ++kap) {
          bf16x8 p;
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = (__bf16)S[8 * kap + e];
          if (kap == 0) {
            u32x4 pb = __builtin_bit_cast(u32x4, p);
            pb[0] |= (vote && lane == 0) ? 0x8000u : 0u;
            p = __builtin_bit_cast(bf16x8, pb);
          }
          lds_store<bf16x8>(pwr + (2 * wave + kap) * 1024 + 16 * lane, p);
        }
#pragma unroll
        for (int idx = 8; idx < 16; ++idx) {
          const int n = idx >> 2, mb = idx & 3;
          if (mb == 0 && n < 3) B[(n + 1) & 1] = p_read(1, n + 1);
          pv_mfma(mb, n);
        }
        {
          float sm[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) sm[i] = S[i] + S[i + 8];
#pragma unroll
          for (int i = 0; i < 4; ++i) sm[i] += sm[i + 4];
          l_run += (sm[0] + sm[1]) + (sm[2] + sm[3]);
        }
      }
      // ---- drain: the latent accumulation of the last sub-tile.  The query
      // registers are free from here on: the next segment's query loads now,
      // under the accumulation and the partial's write.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_barrier();  // P of the last sub-tile (with the votes) is visible
      if (has_next) load_q(nxt.b);
      {
        const int pvb = slot_off(base + nsub - 1) + pa;
        const int prd = kPBufOff + ((nsub + 1) & 1) * kPBufBytes;
        pv_read_at(pvb, 0);
        B[0] = p_read_at(prd, 0, 0);
        pv_build();
        static_for<0, 16>([&](auto ic_) {
          constexpr int idx = decltype(ic_)::value, n = idx >> 2, mb = idx & 3;
          if constexpr (mb == 0)
            B[(n + 1) & 1] = n < 3 ? p_read_at(prd, 0, n + 1) : p_read_at(prd, 1, 0);
          if constexpr (idx == 4) pv_read_at(pvb, 1);
          pv_mfma(mb, n);
          __builtin_amdgcn_sched_barrier(0);
        });
        pv_build();
        static_for<0, 16>([&](auto ic_) {
          constexpr int idx = decltype(ic_)::value, n = idx >> 2, mb = idx & 3;
          if constexpr (mb == 0 && n < 3) B[(n + 1) & 1] = p_read_at(prd, 1, n + 1);
          pv_mfma(mb, n);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // a score more than kLazy above the reference anywhere in the work-group
      // (a vote in the P of the last sub-tile, visible since the drain's
      // barrier): redo the segment with the exact maximum seen in
      // this pass (rare).  The redo starts at the ring position after this
      // pass, behind the loads in flight there (same slots, issued earlier by
      // the same wave, so they land earlier).
      if (mode == 0) {
        const int pv = kPBufOff + ((nsub + 1) & 1) * kPBufBytes;
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v |= lds_load<uint32_t>(pv + 2 * w * 1024);
        // the same word in every lane: a uniform decision
        if (__builtin_amdgcn_readfirstlane(v) & 0x8000u) {
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

    // the window of the segment after the next, issued before the partial's
    // stores so that waiting for it does not wait for the stores
    int pid_n2 = 0;
    if (k + 2 < k_end) {
      const Seg s2 = seg_at(k + 2);
      pid_n2 = load_window(s2.b, s2.t0 / page);
    }

    // ---- unnormalised partial (m, l, o~): o~ rounded to bf16, in register
    // order (8-byte piece 4x + a of a lane holds elements 4a .. 4a + 3 of
    // accumulator x); merged later
    {
      const int ln = lane_here();
      uint2* dst = (uint2*)(part_o + (long)k * kHeads * kDc) + (wave * 64 + ln);
#pragma unroll
      for (int x = 0; x < 16; ++x)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float f0 = acc[x][4 * a], f1 = acc[x][4 * a + 1];
          const float f2 = acc[x][4 * a + 2], f3 = acc[x][4 * a + 3];
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 p0 = {(__bf16)f0, (__bf16)f1}, p1 = {(__bf16)f2, (__bf16)f3};
          dst[(x * 4 + a) * kThreads] =
              uint2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
          // one accumulator at a time: the next query is arriving in the
          // VGPRs, and reading all accumulators ahead would not fit beside it
          if (a == 3) __builtin_amdgcn_sched_barrier(0);
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

// Rows [B][128][576] -> query tiles (qtile_index): one 16-byte piece (eight
// consecutive numbers of one row, which stay consecutive) per thread.
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
  // thread t takes lane tt & 63 of the attention kernel's wave wo = tt >> 6,
  // whose accumulators x = 4 mb + n hold latent dims [128 wo, 128 wo + 128);
  // the two halves of the work-group sum the even and the odd segments
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
    // four segments' loads in flight per half at once; each half sums its
    // segments in order
    constexpr int kU = 4;
    for (int s0 = half; s0 < nc; s0 += 2 * kU) {
      uint2 v[kU][16];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (s0 + 2 * u >= nc) break;
        const uint2* src =
            (const uint2*)(part_o + (long)(k0 + c0 + s0 + 2 * u) * kHeads * kDc) + tt;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int a = 0; a < 4; ++a) v[u][4 * mb + a] = src[((4 * mb + n) * 4 + a) * kThreads];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (s0 + 2 * u >= nc) break;
        const float ws = w[s0 + 2 * u][hd_l];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[r] += ws * f32x4{__uint_as_float(v[u][r].x << 16),
                               __uint_as_float(v[u][r].x & 0xffff0000u),
                               __uint_as_float(v[u][r].y << 16),
                               __uint_as_float(v[u][r].y & 0xffff0000u)};
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
    // (mb, n) at lane (m32, hf) is head 32n + m32, dim 128 wo + 4 (8a + 4 hf + c) + mb
    const int hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          stage[hd_l][128 * wo + 4 * (8 * a + 4 * hf + c) + mb] = (__bf16)acc[4 * mb + a][c];
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
// x = 4 mb + n of the attention kernel's wave wo holds, in element 4a' + c at
// lane (m32, hf), head 32n + m32 and dim 128 wo + 4 (8a' + 4 hf + c) + mb; the
// work-group z = 4 wo + a takes a' = a of all four mb: dims 128 wo + 32 a ..
// + 31, one contiguous run.  Sixteen times the work-groups of
// combine_v2_kernel, so that a few sequences with many segments each still
// spread over the GPU; within a work-group wave q sums the segments
// s = q (mod kRunWaves), the first loads are issued before the softmax
// statistics are formed, and the waves' sums are added at the end in a fixed
// order.
// ---------------------------------------------------------------------------
constexpr int kRunWaves = 4;   // waves per merge work-group, each a share of the segments
constexpr int kRunSegs = 264;   // (m, l) kept in LDS: every automatic plan (<= CUs + 1 segments)

__global__ __launch_bounds__(64 * kRunWaves) void combine_v2_runs_kernel(PlanPtrs plan,
                                                         const __bf16* __restrict__ part_o,
                                                         const float* __restrict__ part_ml,
                                                         __bf16* __restrict__ lat_out) {
  __shared__ float2 s_ml[kRunSegs][32];   // (m, l), then the segment weights in .x
  __shared__ float s_M[32], s_inv[32];
  __shared__ f32x4 s_acc[kRunWaves - 1][4][64];   // the sums of waves 1 ..
  __shared__ __bf16 stage[32][32 + 8];
  const int b = blockIdx.x, n = blockIdx.y, wo = blockIdx.z >> 2, a = blockIdx.z & 3;
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;
  const int cnt = plan.seq_seg_count[b];
  const int k0 = plan.seq_seg_start[b];
  __bf16* out = lat_out + ((long)b * kHeads + n * 32) * kDc + 128 * wo + 32 * a;
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
  uint2 v[kU][4];
  auto issue = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int su = min(s0 + kRunWaves * u, cnt - 1);   // past the end: re-read, weight 0
      const uint2* src =
          (const uint2*)(part_o + (long)(k0 + su) * kHeads * kDc) + wo * 64 + lane;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) v[u][mb] = src[((4 * mb + n) * 4 + a) * kThreads];
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
  f32x4 acc[4];   // [mb]
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
      for (int mb = 0; mb < 4; ++mb)
        acc[mb] += ws * f32x4{__uint_as_float(v[u][mb].x << 16),
                              __uint_as_float(v[u][mb].x & 0xffff0000u),
                              __uint_as_float(v[u][mb].y << 16),
                              __uint_as_float(v[u][mb].y & 0xffff0000u)};
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
    // element c of acc[mb] at lane (m32, hf): head 32n + m32, dim
    // 32 a + 16 hf + 4 c + mb of this work-group's run
    const int hf = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int c = 0; c < 4; ++c) stage[hd_l][16 * hf + 4 * c + mb] = (__bf16)acc[mb][c];
  }
  __syncthreads();
  if (tid < 128) {
    const int hh = tid >> 2, c8 = tid & 3;
    *(uint4*)(out + (long)hh * kDc + 8 * c8) = *(const uint4*)(&stage[hh][8 * c8]);
  }
}

}  // namespace

hipError_t attn_decode_v2(const Geo& g, const void* q_tiles, const void* cache, int num_pages,
                          const int32_t* page_table, int max_pages, const PlanPtrs& plan,
                          int n_wg_launch, void* part_o, float* part_ml, hipStream_t s) {
  if (n_wg_launch <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_v2_kernel, dim3(n_wg_launch), dim3(kThreads), 0, s,
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
