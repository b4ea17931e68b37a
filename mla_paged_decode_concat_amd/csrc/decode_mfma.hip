// Split-KV MLA decode, stage 1, on the gfx950 matrix cores.
//
// What it computes is stage 1 of the split-KV decode of the "fix TP" vLLM
// diff (vllm/attention/ops/triton_decode_attention.py,
// _fwd_grouped_kernel_stage1): for one request's token range and a group of
// heads, scores s = sm_scale * q . row over the full R+P row, an online
// softmax, values = the first R columns of the same rows, and the stored
// partial (acc / l, m + ln l) in the fp32 workspace (the pages size it as
// [B, H, S, R+1]; the slot layout here is this library's own: partial rows
// [H, slots, R], then the LSEs [H, slots]).
//
// How (MI355X-first, not the pages' Triton tiling):
//  * One workgroup owns a token range and up to 128 heads, so each 32-token
//    KV tile is read from HBM once and shared by every head (the Triton
//    prior art re-reads it per 16-head group).
//  * Tiles stream HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//    STAGES tiles in flight; an fp8 cache's tiles are read by the matrix
//    cores as fp8 and converted to bf16 in registers.  Inside a tile, 8 tokens x 128 bytes (full
//    cache lines) form one 1 KB block written by one load instruction; the
//    slot swizzle 8*t + (c ^ (2*(t >> 1) + (tq & 1))) keeps both LDS read
//    patterns below free of bank conflicts.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16: A = K rows from LDS
//    (ds_read_b128), B = Q^T kept in registers for the whole range.
//  * O^T = V^T P^T: A = V^T via ds_read_b64_tr_b16 (4 tokens x 1 column per
//    lane), B = P^T taken straight from the S^T accumulators: the MFMA
//    result layout (lane = head, 4 consecutive tokens per lane group) is the
//    B-operand layout once the 8 k-slots of a lane are bound to tokens
//    {4g..4g+3, 16+4g..16+4g+3}.  Every per-head quantity therefore lives in
//    the lane that owns the head; nothing moves across lanes per tile.
//  * Fixed softmax reference: each head's reference is set on the first tile
//    of a pass and p = 2^(s - ref) is accumulated unscaled; a tile more than
//    32 (log2 units) above the reference makes the workgroup redo its range
//    with the larger reference.  acc and l always share the reference, so the
//    result is the exact softmax, and acc is never multiplied (which keeps it
//    in the accumulation registers).
//  * Each CU keeps only about 36-40 KB of loads in flight before a further
//    load issue stalls the issuing wave, so a workgroup gets about one tile
//    per HBM round trip.  With four waves, each issues its loads of the tile
//    three ahead at its own point of PV; narrower workgroups issue theirs in
//    two parts, after the tile barrier and after QK.
//  * Workgroups of 16 or 32 heads are one wave with a two-tile ring, several
//    to a CU (one wave per SIMD), so their stalls and compute overlap.
//  * The request's block-table slice is staged in LDS, so page lookups are
//    LDS reads and never wait behind the tile loads on the vmcnt counter.
//  * Workgroups that share a token range (different head groups) get ids
//    that the dispatcher sends to the same XCD, so their common KV tiles
//    meet in that XCD's L2.
#include "mla_device.h"
#include "mla_launch.h"

#include <type_traits>
#include <utility>

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MLA_LDS(T, ptr) ((__attribute__((address_space(3))) T*)(ptr))

constexpr int kTile = 32;            // tokens per KV tile
constexpr int kTableWindow = 1024;   // block-table entries staged in LDS
constexpr int kXcds = 8;             // MI355X: workgroup i runs on XCD i % 8
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 32.0f;        // log2 units: p = 2^(s - m_ref) stays below 2^32

template <int R>
struct Geo {
  static constexpr int D = R + 64;
  static constexpr int ROW_BYTES = D * 2;          // bf16 row
  static constexpr int CHUNKS = ROW_BYTES / 16;    // 16-byte chunks per row
  static constexpr int NBLK = CHUNKS / 4 * 2;      // 1 KB blocks per tile
  static constexpr int TILE_BYTES = NBLK * 1024;
  static constexpr int KS = D / 32;                // QK k-steps of 32
  static constexpr int CB = R / 16;                // PV column blocks of 16
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16 bytes per lane HBM -> LDS (global_load_lds_dwordx4): lane i reads
// gptr + OFF and its bytes land at LDS address lds_base + 16 * i.  The
// instruction's immediate offset is added to the LDS address too (M0 + OFF +
// 16 i), so M0 is set to lds_base - OFF; callers keep lds_base >= OFF.  The
// ISA asks for one wait state between writing M0 and the load; M0 is
// declared clobbered, so the compiler keeps nothing of its own there.  Issued
// through inline asm so the compiler does not add a full vmcnt drain before
// every later LDS read (it cannot prove the in-flight tile and the tile being
// read are disjoint); the kernel orders them itself with wait_vmcnt + a
// workgroup barrier.
//
// NT sets the load's non-temporal hint (a compile-time choice: a branch
// around every load instruction slowed the one-wave kernels by half): the lines are not
// expected to be read again, so they do not displace reusable data in L2
// and the last-level cache.  That holds when one or two head groups read
// each tile; tiles shared by more groups meet in L2 and are loaded without
// it.  Measured on the V3 shape (128 heads, one group): stage 1 172 -> 161
// us, and stage 2, which reads the partials that stage 1 leaves in the
// caches, 17.7 -> 17.0 us; two query tokens per request (two 128-row
// groups) 327 -> 316 us.
template <int OFF, bool NT>
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset");
  // M0 (the LDS destination) is an input operand: the compiler writes it
  // and knows its value; the s_nop separates that write from the load
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base - OFF);
  if constexpr (NT)
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2 nt" ::"v"(gptr), "{m0}"(m0), "i"(OFF)
                 : "memory");
  else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(gptr), "{m0}"(m0), "i"(OFF)
                 : "memory");
}

// This lane's index, read so that the compiler cannot hoist what is derived
// from it out of a loop: per-lane address terms are then recomputed (a few
// instructions) instead of being kept live across the tile loop, where they
// would push the register budget over and get spilled (a scratch reload
// waits on the same counter as the tile loads in flight).
__device__ __forceinline__ int lane_now() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The workgroup thread index formed the same way (wave index in a scalar
// register, lane through lane_now()), for the strided loops that stage the
// block table or clear an empty request's output: their per-thread addresses
// are then formed where the loop runs instead of at kernel entry.
__device__ __forceinline__ int tid_now() {
  return (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * kWave + lane_now();
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)MLA_LDS(const char, p);
}

typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (bytes of w0, then w1) -> 8 bf16, exactly: an E4M3 value has
// 4 significant bits, and the conversion's scale is 1
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1
template <class F, int... I>
__device__ __forceinline__ void static_for_(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_(f, std::make_integer_sequence<int, N>{});
}

// Tile loads.  Tile layout in LDS: block (cq8, tq) = chunks 8*cq8 .. +7 (16
// bytes each) of tokens 8*tq .. +7, at byte (4*cq8 + tq) * 1024; inside it
// token t8, chunk c8 sits in 16-byte slot 8*t8 + (c8 ^ swz(t8, tq)).  One
// load instruction fills one block: lane i takes token i / 8 and the chunk
// whose slot is i, so each group of 8 lanes reads one full 128-byte line.
// With NW waves sharing a tile, wave w loads token quarters w, w + NW, ...;
// its load i fills block (cq8 = i / NQ, tq = w + NW * (i % NQ)), from one
// per-quarter lane address plus the immediate offset 128 * cq8 (the block
// sits at 1024 * (4 cq8 + tq) >= 128 cq8 bytes, as dma16 requires).
template <int R, int NW>
struct TileLoad {
  using G = Geo<R>;
  static_assert(NW == 1 || NW == 2 || NW == 4, "waves per tile");
  static constexpr int NQ = 4 / NW;                // token quarters per wave
  static constexpr int LPW = G::NBLK / NW;         // load instructions per wave per tile
  static_assert(G::NBLK % NW == 0, "tile blocks must split evenly over the waves");
  static __device__ __forceinline__ int swz(int t8, int tq) { return 2 * (t8 >> 1) + (tq & 1); }

  struct Rows {
    const char* r[NQ];
  };
  static __device__ __forceinline__ Rows rows(const DecodeParams& p, int tile_start, int se, int pg0,
                                              const int* s_table, int wave) {
    const char* cache = reinterpret_cast<const char*>(p.cache);
    const int lane = lane_now();
    const int t8 = lane >> 3, x = lane & 7;
    Rows rw;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int tq = wave + NW * j;
      int tok = tile_start + 8 * tq + t8;
      tok = tok < se ? tok : se - 1;              // past the range: re-read a valid row (masked later)
      int pg, row;
      page_split(p, tok, pg, row);
      const long long page = s_table[pg - pg0];
      rw.r[j] = cache + (page * p.block_stride + (long long)row * G::D) * 2 + (x ^ swz(t8, tq)) * 16;
    }
    return rw;
  }
  // a tile's column groups cq8 < CQ-1 (values) go to vbuf, the last (rope) to rbuf
  static constexpr int CQ = G::CHUNKS / 8;
  template <int I, bool NT>
  static __device__ __forceinline__ void issue(const Rows& rw, const char* vbuf, const char* rbuf, int wave) {
    constexpr int j = I % NQ, cq8 = I / NQ;
    if constexpr (cq8 < CQ - 1)
      dma16<128 * cq8, NT>(rw.r[j], lds_addr(vbuf) + (wave + NW * j + 4 * cq8) * 1024);
    else
      dma16<128 * cq8, NT>(rw.r[j], lds_addr(rbuf) + (wave + NW * j) * 1024);
  }
  template <bool NT>
  static __device__ __forceinline__ void tile(const DecodeParams& p, int tile_start, int se, int pg0,
                                              const char* vbuf, const char* rbuf, const int* s_table, int wave,
                                              int lane) {
    const Rows rw = rows(p, tile_start, se, pg0, s_table, wave);
    static_for<LPW>([&](auto i) { issue<decltype(i)::value, NT>(rw, vbuf, rbuf, wave); });
  }
};

// fp8 E4M3 cache tiles.  A 32-token tile holds, per token quarter tq, the
// value columns as R/128 full blocks (cq8, tq) of 8 tokens x 128 bytes at
// (4 cq8 + tq) * 1024 (token t8, 16-byte chunk c8 at slot 8 t8 + (c8 ^ t8)),
// and the 64 rope bytes as a half block at ROPE_OFF + tq * 512 (token t8,
// chunk y at slot 4 t8 + ((y + t8 / 2) & 3)).  The swizzles spread the 8
// tokens of a block over all eight 16-byte bank groups for both read
// patterns below.  Loads of a full block are one LDS-DMA instruction (each
// 8-lane group reads one 128-byte line); the rope half block is one
// instruction with the upper 32 lanes masked off (their LDS destinations
// would lie past the half block).  The matrix cores read the fp8 tile
// directly: K fragments as 16 contiguous bytes per lane, V^T fragments with
// the 8-bit transpose read, each converted to bf16 in registers (exactly).
template <int R, int NW>
struct TileLoad8 {
  static constexpr int D = R + 64;
  static constexpr int FG = R / 128;                 // full 128-byte groups (the value columns)
  static constexpr int NQ = 4 / NW;                  // token quarters per wave
  static constexpr int LPW = NQ * (FG + 1);          // load instructions per wave per tile
  static constexpr int ROPE_OFF = FG * 4096;
  static constexpr int TILE_BYTES = ROPE_OFF + 4 * 512;
  static constexpr int CPR = D / 16;                 // 16-byte chunks per row

  struct Rows {
    const char* full[NQ];
    const char* rope[NQ];
  };
  static __device__ __forceinline__ const char* row_ptr(const DecodeParams& p, int tok, int se, int pg0,
                                                        const int* s_table) {
    tok = tok < se ? tok : se - 1;                 // past the range: re-read a valid row (masked later)
    int pg, row;
    page_split(p, tok, pg, row);
    const long long page = s_table[pg - pg0];
    return reinterpret_cast<const char*>(p.cache) + page * p.block_stride + (long long)row * D;
  }
  static __device__ __forceinline__ Rows rows(const DecodeParams& p, int tile_start, int se, int pg0,
                                              const int* s_table, int wave) {
    const int lane = lane_now();
    Rows rw;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int tq = wave + NW * j;
      // lane i fills slot i: token i / 8, chunk (i % 8) ^ token
      rw.full[j] = row_ptr(p, tile_start + 8 * tq + (lane >> 3), se, pg0, s_table) + ((lane & 7) ^ (lane >> 3)) * 16;
      // rope lane i < 32 fills slot i: token t = i / 4, chunk (i % 4 - t / 2) & 3
      const int tr = (lane & 31) >> 2;
      rw.rope[j] = row_ptr(p, tile_start + 8 * tq + tr, se, pg0, s_table) + R + (((lane & 3) - (tr >> 1)) & 3) * 16;
    }
    return rw;
  }
  template <int I, bool NT>
  static __device__ __forceinline__ void issue(const Rows& rw, const char* buf, int wave, int lane) {
    constexpr int j = I / (FG + 1), k = I % (FG + 1);
    const int tq = wave + NW * j;
    if constexpr (k < FG) {
      dma16<128 * k, NT>(rw.full[j], lds_addr(buf) + (4 * k + tq) * 1024);
    } else {
      if (lane < 32) dma16<0, NT>(rw.rope[j], lds_addr(buf) + ROPE_OFF + tq * 512);
    }
  }
  template <bool NT>
  static __device__ __forceinline__ void tile(const DecodeParams& p, int tile_start, int se, int pg0,
                                              const char* buf, const int* s_table, int wave, int lane) {
    const Rows rw = rows(p, tile_start, se, pg0, s_table, wave);
    static_for<LPW>([&](auto i) { issue<decltype(i)::value, NT>(rw, buf, wave, lane); });
  }

};

template <int R, int NB, int NW, int STAGES, bool F8 = false>
struct Stage1 {
  using G = Geo<R>;
  using TL8 = TileLoad8<R, NW>;
  // DMA instructions per wave per tile
  static constexpr int LPW = F8 ? TL8::LPW : G::NBLK / NW;
  static_assert(G::NBLK % NW == 0, "tile blocks must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");
  static constexpr int HPG = 16 * NB * NW;         // heads per workgroup
  static constexpr int NW_ = NW;
  // ring slot per tile in flight
  static constexpr int SLOT = F8 ? TL8::TILE_BYTES : G::TILE_BYTES;
  static constexpr int SMEM = STAGES * SLOT;
  static constexpr int TABLE = kTableWindow;       // block-table window staged in LDS

  // wait until the loads of the tile that has `after` newer tiles in flight landed
  static __device__ __forceinline__ void wait_tile(int after) {
    if constexpr (STAGES >= 4) {
      if (after >= 2) { wait_vmcnt<2 * LPW>(); return; }
    }
    if constexpr (STAGES >= 3) {
      if (after >= 1) { wait_vmcnt<LPW>(); return; }
    }
    wait_vmcnt<0>();
  }

  static __device__ __forceinline__ int swz(int t8, int tq) { return TileLoad<R, NW>::swz(t8, tq); }
  // bf16 tiles, one or two waves: load instructions issued before QK; the rest follow QK
  static constexpr int kFirst = (LPW * 5 + 8) / 9;
  // bf16 tiles, four waves: each wave issues all of its loads for the tile
  // three ahead at its own PV column block (1/16, 5/16, 9/16 and 13/16 of
  // the way through PV), so that the four bursts do not queue behind each
  // other at the CU's load unit and none of them stalls QK, whose K reads
  // are the denser LDS stream.  (Measured against two points in QK and two
  // in PV: 156.0 vs 161.9 us, faster in 15 of 16 interleaved rounds.)
  // Points are encoded as 100 + QK k-step or 300 + PV column block.
  static constexpr bool kStagger = !F8 && NW == 4;
  static constexpr int kIssueAt[4] = {300 + G::CB / 16, 300 + G::CB * 5 / 16, 300 + G::CB * 9 / 16,
                                      300 + G::CB * 13 / 16};
  template <int I, bool NT>
  static __device__ __forceinline__ void issue_part(const typename TileLoad<R, NW>::Rows& rw, char* buf, int wave) {
    TileLoad<R, NW>::template issue<I, NT>(rw, buf, buf + (G::CHUNKS / 8 - 1) * 4096, wave);
  }
  template <bool NT>
  static __device__ __forceinline__ void issue_tile(const DecodeParams& p, int tile_start, int se, int pg0,
                                                    char* buf, const int* s_table, int wave, int lane) {
    if constexpr (F8)
      TL8::template tile<NT>(p, tile_start, se, pg0, buf, s_table, wave, lane);
    else
      TileLoad<R, NW>::template tile<NT>(p, tile_start, se, pg0, buf, buf + (G::CHUNKS / 8 - 1) * 4096, s_table, wave,
                                         lane);
  }

  // Token range [a, e) of request b for this wave's heads; writes partial
  // slot `part`.  NT: the tile loads carry the non-temporal hint.
  template <bool NT>
  static __device__ void piece(const DecodeParams& p, int b, int a, int e, int part, int head0,
                               char* smem, int* s_table, int* s_flags) {
    const int lane = lane_now();   // per-lane terms formed per piece, not at kernel entry
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int r16 = lane & 15;
    head0 += wave * 16 * NB;                   // this wave's heads

    // an fp8 cache stores row / kv_scale: the scale goes into the scores and the output
    const float kvs = F8 ? *p.kv_scale : 1.0f;
    // ---- Q^T operand in registers: lane = head r16 of block nb, dims 32ks + 8g .. +8
    // (fp8 cache: k-step pair kp = ks / 2 covers dims 64kp .. +64, of which
    // lane group g takes 64kp + 16g .. +16, half ks % 2 in k-step ks -- the
    // K fragments then come from 16 contiguous bytes per lane)
    bf16x8_t qf[NB][G::KS];
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (long long)b * p.q_sb;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = head0 + 16 * nb + r16;     // head groups divide H: always a real head
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        const int d = F8 ? 64 * (ks >> 1) + 16 * g + 8 * (ks & 1) : 32 * ks + 8 * g;
        qf[nb][ks] = *reinterpret_cast<const bf16x8_t*>(qb + (long long)h * p.q_sh + d);
      }
    }
    // Q is waited for after the block table's first window is staged (its
    // loads are in flight together with Q's), before the tile loop.

    f32x4_t acc[G::CB][NB];
    // l_sum: the exact sum of p (for the LSE); l_mma: the sum of p as rounded
    // to bf16 for the matrix cores, which normalises acc.  The normalised
    // weights then sum to one exactly, so the rounding of a dominant weight
    // cancels instead of scaling the output by up to 2^-9.  With an fp8 cache
    // the matrix cores take p as bf16 plus its bf16 remainder, which together
    // are within 2^-17 of p, so l_sum normalises acc as well.
    float m_ref[NB], l_sum[NB], l_mma[NB], m_init[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) m_init[nb] = -INFINITY;
    const float c2 = p.sm_scale * kvs * kLog2e;

    // lane-constant LDS offsets
    // K rows (A operand of QK): token m = r16 of a 16-token block, chunk 4ks + g;
    // k_off[ks & 1] is the lane part, the block part is compile-time
    uint32_t k_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int t8 = r16 & 7, tqo = r16 >> 3, c8 = 4 * par + g;
      k_off[par] = (uint32_t)(tqo * 1024 + (8 * t8 + (c8 ^ swz(t8, tqo))) * 16);
    }
    // V^T (A operand of PV) via transpose reads: this lane addresses token
    // 16tb + 4g + (r16 >> 2), bytes [8 * (r16 & 3), +8) of a 16-column block;
    // v_off[cb & 3] is the lane part
    uint32_t v_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sg = r16 & 3;
      const int t8 = 4 * (g & 1) + (r16 >> 2), tqo = g >> 1;
      const int c8 = 2 * k + (sg >> 1);
      v_off[k] = (uint32_t)(tqo * 1024 + (8 * t8 + (c8 ^ swz(t8, tqo))) * 16 + (sg & 1) * 8);
    }
    const int bs = p.block_size;
    const int32_t* btab = p.block_table + (long long)b * p.bt_stride;

    // Softmax reference: each head's running max is fixed on the first tile
    // of the pass (the accumulators are still zero there, so nothing is
    // rescaled) and p = 2^(s - m_ref) is accumulated unscaled after that.  A
    // later tile more than kSlack above the reference cannot be represented;
    // then the workgroup finishes the tile, drops the pass and redoes the
    // range with the larger reference.  Each redo raises a reference by more
    // than kSlack, so this terminates; on real attention scores it does not
    // happen.  The accumulators are never multiplied, which keeps them in
    // the accumulation registers.
#pragma unroll 1
    for (;;) {
#pragma unroll
      for (int cb = 0; cb < G::CB; ++cb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        m_ref[nb] = m_init[nb];
        l_sum[nb] = 0.0f;
        l_mma[nb] = 0.0f;
      }
      bool redo = false;

      for (int sa = a; sa < e && !redo;) {
        const int pg0 = sa / bs;
        const long long win_end = (long long)(pg0 + kTableWindow) * bs;
        int se = e;
        if (win_end < e) se = sa + (int)((win_end - sa) / kTile) * kTile;
        __syncthreads();   // earlier readers of s_table, s_flags and the tile buffers are done
        const int npg = (se - 1) / bs - pg0 + 1;
        for (int i = tid_now(); i < npg; i += NW * 64) s_table[i] = btab[pg0 + i];
        if (threadIdx.x == 0) {
          s_flags[0] = 0;
          s_flags[1] = 0;
        }
        // Q (loaded at the top of the piece) and the table have landed before
        // the tile loop: without this the compiler guards each first use of Q
        // inside the loop with a vmcnt wait, which would also drain the tile
        // loads in flight on every iteration.
        wait_vmcnt<0>();
        __syncthreads();

        const int ntiles = (se - sa + kTile - 1) / kTile;
#pragma unroll
        for (int t = 0; t < STAGES - 1; ++t)
          if (t < ntiles) issue_tile<NT>(p, sa + kTile * t, se, pg0, smem + t * SLOT, s_table, wave, lane);

#pragma unroll 1
        for (int t = 0; t < ntiles; ++t) {
          const int after = min(STAGES - 2, ntiles - 1 - t);
          wait_tile(after);
          __syncthreads();   // tile t landed in every wave; tile t-1's buffer is free
          // a redo flagged while computing tile t-1 is seen by all waves here
          if (t > 0 && s_flags[(t - 1) & 1]) {
            redo = true;
            break;
          }
          // Tile t + STAGES - 1 into the buffer tile t - 1 used.  bf16: about
          // five ninths of a wave's load instructions go out here and the rest
          // after QK, so that the waves do not all stall on one burst (measured
          // 3-4% faster on the V3 shape than a single burst).
          const bool more = t + STAGES - 1 < ntiles;
          char* nbuf = smem + ((t + STAGES - 1) % STAGES) * SLOT;
          typename TileLoad<R, NW>::Rows nrw;
          if constexpr (F8) {
            if (more) issue_tile<NT>(p, sa + kTile * (t + STAGES - 1), se, pg0, nbuf, s_table, wave, lane);
          } else if constexpr (!kStagger) {
            if (more) {
              nrw = TileLoad<R, NW>::rows(p, sa + kTile * (t + STAGES - 1), se, pg0, s_table, wave);
              static_for<kFirst>([&](auto i) { issue_part<decltype(i)::value, NT>(nrw, nbuf, wave); });
            }
          }
          // the staggered issue: called at every point, issues in the wave whose point it is
          auto issue_at = [&](auto P) {
            constexpr int pt = decltype(P)::value;
            if constexpr (kStagger) {
              constexpr int wmask = (kIssueAt[0] == pt ? 1 : 0) | (kIssueAt[1] == pt ? 2 : 0) |
                                    (kIssueAt[2] == pt ? 4 : 0) | (kIssueAt[3] == pt ? 8 : 0);
              if constexpr (wmask != 0) {
                if (more && ((wmask >> wave) & 1)) {
                  const typename TileLoad<R, NW>::Rows rw =
                      TileLoad<R, NW>::rows(p, sa + kTile * (t + STAGES - 1), se, pg0, s_table, wave);
                  static_for<LPW>([&](auto i) { issue_part<decltype(i)::value, NT>(rw, nbuf, wave); });
                }
              }
            }
          };
          const char* tile = smem + (t % STAGES) * SLOT;
          const int tile_start = sa + kTile * t;

          // ---- S^T = K Q^T  (2 token blocks x NB head blocks); K rows read two
          // k-steps ahead through a 3-slot ring, one k-step per scheduling region
          f32x4_t s[2][NB];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if constexpr (!F8) {
            bf16x8_t kr[3][2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int mb = 0; mb < 2; ++mb)
                kr[ks][mb] = *MLA_LDS(const bf16x8_t, tile + ((ks >> 1) * 4 + 2 * mb) * 1024 + k_off[ks & 1]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<G::KS>([&](auto KSI) {
              constexpr int ks = decltype(KSI)::value;
              issue_at(std::integral_constant<int, 100 + ks>{});
              if (ks + 2 < G::KS) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                  kr[(ks + 2) % 3][mb] =
                      *MLA_LDS(const bf16x8_t, tile + (((ks + 2) >> 1) * 4 + 2 * mb) * 1024 + k_off[ks & 1]);
              }
#pragma unroll
              for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                  s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % 3][mb], qf[nb][ks], s[mb][nb], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            });
          } else {
            // K fragments straight from the fp8 tile: for k-step pair kp and
            // token block mb, lane (token r16, group g) reads the 16 bytes of
            // dims 64kp + 16g .. +16 and converts them to the bf16 fragments
            // of k-steps 2kp and 2kp + 1; reads run one pair ahead
            constexpr int KP = G::KS / 2;
            constexpr int VP = R / 64;                // pairs in the value columns
            const int t8 = r16 & 7;
            auto kread = [&](int kp, int mb) -> u32x4_t {
              const int tq = 2 * mb + (r16 >> 3);
              const char* a = kp < VP
                                  ? tile + (4 * (kp >> 1) + tq) * 1024 + (8 * t8 + ((4 * (kp & 1) + g) ^ t8)) * 16
                                  : tile + TL8::ROPE_OFF + tq * 512 + (4 * t8 + ((g + (t8 >> 1)) & 3)) * 16;
              return *MLA_LDS(const u32x4_t, a);
            };
            u32x4_t kw[2][2];
            kw[0][0] = kread(0, 0);
            kw[0][1] = kread(0, 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kp = 0; kp < KP; ++kp) {
              if (kp + 1 < KP) {
                kw[(kp + 1) & 1][0] = kread(kp + 1, 0);
                kw[(kp + 1) & 1][1] = kread(kp + 1, 1);
              }
#pragma unroll
              for (int mb = 0; mb < 2; ++mb) {
                const u32x4_t w = kw[kp & 1][mb];
                const bf16x8_t k0 = fp8x8_to_bf16(w[0], w[1]);
                const bf16x8_t k1 = fp8x8_to_bf16(w[2], w[3]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                  s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[nb][2 * kp], s[mb][nb], 0, 0, 0);
                  s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[nb][2 * kp + 1], s[mb][nb], 0, 0, 0);
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }

          if constexpr (!F8 && !kStagger) {
            if (more)
              static_for<LPW - kFirst>([&](auto i) { issue_part<kFirst + decltype(i)::value, NT>(nrw, nbuf, wave); });
          }
          // ---- softmax in the log2 domain; lane owns head r16, tokens 16mb + 4g + i
          bool need = false;
          float mt[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            mt[nb] = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int tok = tile_start + 16 * mb + 4 * g + i;
                const float v = tok < se ? s[mb][nb][i] * c2 : -INFINITY;
                s[mb][nb][i] = v;
                mt[nb] = fmaxf(mt[nb], v);
              }
            need |= mt[nb] > m_ref[nb] + kSlack;    // also true while m_ref is unset (-inf)
          }
          if (__builtin_expect(__any(need), 0)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              float m = mt[nb];
              m = fmaxf(m, __shfl_xor(m, 16, 64));
              m = fmaxf(m, __shfl_xor(m, 32, 64));
              if (m_ref[nb] == -INFINITY) {
                m_ref[nb] = m;                     // first tile of the pass
              } else if (m > m_ref[nb] + kSlack) {
                m_init[nb] = m;                    // not representable in this pass
                s_flags[t & 1] = 1;
              }
            }
          }
          // P for the matrix cores in bf16.  An fp8 cache also gets the
          // rounding remainder p - bf16(p) as a second bf16 operand (pl): the
          // value columns are then summed against p to ~16 significant bits.
          // A weight rounded to bf16 alone is off by up to 2^-9 of itself,
          // which moves o by up to ~2^-9 |v_j - o| per dominant token; with
          // the wider values an fp8 cache holds that reached the 1e-2 bound.
          bf16x8_t pf[NB], pl[F8 ? NB : 1];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            float ls = 0.0f, lm = 0.0f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pj = __builtin_amdgcn_exp2f(s[mb][nb][i] - m_ref[nb]);
                const __bf16 pb = (__bf16)pj;
                ls += pj;
                pf[nb][4 * mb + i] = pb;
                if constexpr (F8) {
                  pl[nb][4 * mb + i] = (__bf16)(pj - (float)pb);
                } else {
                  lm += (float)pb;
                }
              }
            l_sum[nb] += ls;
            l_mma[nb] += F8 ? ls : lm;
          }

          // ---- O^T += V^T P^T  (CB column blocks x NB head blocks); V^T read
          // two column blocks ahead through a 3-slot ring
          if constexpr (!F8) {
            auto vread = [&](int cb) -> bf16x8_t {
              const char* vb = tile + (cb >> 2) * 4096 + v_off[cb & 3];
              const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, vb));
              const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, vb + 2048));
              return bf16x8_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            };
            __builtin_amdgcn_sched_barrier(0);
            bf16x8_t vr[3];
            vr[0] = vread(0);
            vr[1] = vread(1);
            __builtin_amdgcn_sched_barrier(0);
            static_for<G::CB>([&](auto CBI) {
              constexpr int cb = decltype(CBI)::value;
              issue_at(std::integral_constant<int, 300 + cb>{});
              if (cb + 2 < G::CB) vr[(cb + 2) % 3] = vread(cb + 2);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[cb % 3], pf[nb], acc[cb][nb], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            });
          } else {
            // V^T fragments by the 8-bit transpose read: in lane group g,
            // source lane r16 = 2i + hh names the token bound to k-slot i
            // ({4g .. 4g+3, 16+4g .. 16+4g+3}) and byte half hh of a 16-column
            // block; lane (g, c) gets column c of those 8 tokens
            const int i8 = r16 >> 1, hh = r16 & 1;
            const int tok = i8 < 4 ? 4 * g + i8 : 12 + 4 * g + i8;
            const int tqv = tok >> 3, t8v = tok & 7;
            auto vread8 = [&](int cb) -> v2i32_t {
              const char* a = tile + (4 * (cb >> 3) + tqv) * 1024 + (8 * t8v + ((cb & 7) ^ t8v)) * 16 + 8 * hh;
              return __builtin_amdgcn_ds_read_tr8_b64_v2i32(MLA_LDS(v2i32_t, a));
            };
            __builtin_amdgcn_sched_barrier(0);
            v2i32_t vw[3];
            vw[0] = vread8(0);
            vw[1] = vread8(1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int cb = 0; cb < G::CB; ++cb) {
              if (cb + 2 < G::CB) vw[(cb + 2) % 3] = vread8(cb + 2);
              const bf16x8_t vf = fp8x8_to_bf16((uint32_t)vw[cb % 3][0], (uint32_t)vw[cb % 3][1]);
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[nb], acc[cb][nb], 0, 0, 0);
                acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[nb], acc[cb][nb], 0, 0, 0);
              }
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
        if (!redo) {
          __syncthreads();   // a redo flagged on the last tile
          redo = s_flags[(ntiles - 1) & 1] != 0;
        }
        wait_vmcnt<0>();     // nothing may still be landing when the buffers are reused
        sa = se;
      }
      if (!redo) break;
    }

    // ---- finalize: l over the 4 lanes sharing a head, normalise, store the partial
    // (the lane is read again here so that the store addresses are worked out
    // after the tile loop, not hoisted into registers the loop holds or spills)
    const int lane_f = lane_now();
    const int gf = lane_f >> 4, rf = lane_f & 15;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l = l_sum[nb], lm = l_mma[nb];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
      lm += __shfl_xor(lm, 16, 64);
      lm += __shfl_xor(lm, 32, 64);
      const float inv = kvs / lm;
      const float lse = (m_ref[nb] + __builtin_amdgcn_logf(l)) * kLn2;
      const int h = head0 + 16 * nb + rf;
      if (p.direct) {   // one branch for the whole row, not one per store
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb) {
          const f32x4_t v = acc[cb][nb] * inv;
          store_partial4<true>(p, b, part, h, R, 16 * cb + 4 * gf, v[0], v[1], v[2], v[3]);
        }
      } else {
#pragma unroll
        for (int cb = 0; cb < G::CB; ++cb) {
          const f32x4_t v = acc[cb][nb] * inv;
          store_partial4<false>(p, b, part, h, R, 16 * cb + 4 * gf, v[0], v[1], v[2], v[3]);
        }
      }
      if (gf == 0) store_partial_lse(p, b, part, h, R, lse);
    }
  }
};

// Stage 1 for a 128-head group on a bf16 cache, with two waves per SIMD in
// different roles.  One wave per SIMD cannot keep its SIMD's matrix core busy:
// its LDS reads wait out their latency, its softmax leaves the matrix core
// idle, and a tile-load issue that finds the CU's load queue full stalls it.
// Here SIMD j runs two waves for the 32 heads 32j .. 32j+31:
//  * the QK wave (waves 0-3) holds Q for its heads in registers, computes
//    S^T = K Q^T over the tile, the softmax (fixed reference, as in Stage1),
//    writes P (bf16, the matrix cores' B-operand layout) to LDS and
//    accumulates value columns 0 .. 16*CA-1 itself;
//  * the PV wave (waves 4-7) accumulates the other value columns, one tile
//    behind: in the interval in which the QK wave works on tile k it reads
//    P(k-1) and tile k-1's V^T, and it issues all of the tile loads (its
//    token quarter of tile k+2), so a stalled load issue never holds up the
//    QK chain.
// While one wave of a SIMD runs vector code or waits on LDS the other one
// feeds the matrix core.  One workgroup barrier per tile orders everything:
// after barrier k, tile k has landed, P(k-1) is written, and the ring slots
// of tiles k-2 (values) and k-1 (rope columns) are free.  The value columns
// of a tile sit in a 4-slot ring (read by the QK wave in interval k and by
// the PV wave in interval k+1), the rope columns in a 3-slot ring (QK only).
// Every head's accumulation order is the one Stage1 uses, so the results are
// the same bits.
template <int R, int CA, int KRING = 3, int VRA = 3, int VRB = 3>
struct Stage1AB {
  using G = Geo<R>;
  using TL = TileLoad<R, 4>;
  static constexpr int NW_ = 8;
  static constexpr int HPG = 128;
  static constexpr int CB = G::CB;                 // value column blocks of 16
  static constexpr int CBB = CB - CA;              // the PV wave's share
  static_assert(CA >= 1 && CBB >= 1, "column split");
  static constexpr int LPW = G::NBLK / 4;          // load instructions per PV wave per tile
  static constexpr int VKS = R / 32;               // QK k-steps over the value columns
  static constexpr int VSLOT = (G::CHUNKS / 8 - 1) * 4096;
  static constexpr int RSLOT = 4096;
  static constexpr int NV = 4, NR = 3;
  static constexpr int P_OFF = NV * VSLOT + NR * RSLOT;
  static constexpr int PBUF = HPG * kTile * 2;     // P of one tile, bf16
  static constexpr int SMEM = P_OFF + 2 * PBUF;
  static constexpr int TABLE = R == 512 ? 1016 : kTableWindow;
  // LDS read-ahead depths (ring slots): K rows in QK, V^T in each wave's PV
  static constexpr int kKRing = KRING, kVRingA = VRA, kVRingB = VRB;
  static_assert(SMEM + TABLE * 4 + 8 <= 160 * 1024, "LDS");

  static __device__ __forceinline__ char* vslot(char* smem, int t) { return smem + (t % NV) * VSLOT; }
  static __device__ __forceinline__ char* rslot(char* smem, int t) { return smem + NV * VSLOT + (t % NR) * RSLOT; }
  static __device__ __forceinline__ char* pbuf(char* smem, int t, int hg) {
    return smem + P_OFF + (t & 1) * PBUF + hg * 2048;
  }

  template <bool NT>
  static __device__ __forceinline__ void issue(const DecodeParams& p, int sa, int t, int se, int pg0, char* smem,
                                               const int* s_table, int hg) {
    const typename TL::Rows rw = TL::rows(p, sa + kTile * t, se, pg0, s_table, hg);
    char* vb = vslot(smem, t);
    char* rb = rslot(smem, t);
    static_for<LPW>([&](auto i) { TL::template issue<decltype(i)::value, NT>(rw, vb, rb, hg); });
  }

  template <bool NT>
  static __device__ void piece(const DecodeParams& p, int b, int a, int e, int part, int head0,
                               char* smem, int* s_table, int* s_flags) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4) run<true, NT>(p, b, a, e, part, head0, wave, smem, s_table, s_flags);
    else run<false, NT>(p, b, a, e, part, head0, wave - 4, smem, s_table, s_flags);
  }

  // QK wave, one tile: S^T = K Q^T, the softmax, P(k) to LDS for the PV
  // wave, and this wave's own value columns.  Returns nothing; updates the
  // softmax state and may flag a redo.
  template <int KR>
  static __device__ __forceinline__ void qk_tile(const bf16x8_t (&qf)[2][G::KS], f32x4_t (&acc)[CA][2],
                                                 float (&m_ref)[2], float (&l_sum)[2], float (&l_mma)[2],
                                                 float (&m_init)[2], const char* vt, const char* rt, char* pb,
                                                 int tile_start, int se, float c2, int* flag) {
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    // K rows: token r16 of a 16-token block, chunk 4 * (ks & 1) + g of the
    // block's 8 column chunks (swizzled); the block part is an immediate
    const int t8 = r16 & 7, tqo = r16 >> 3;
    const uint32_t k0 = lds_addr(vt) + (uint32_t)(tqo * 1024 + (8 * t8 + ((g) ^ TL::swz(t8, tqo))) * 16);
    const uint32_t k1 = lds_addr(vt) + (uint32_t)(tqo * 1024 + (8 * t8 + ((4 + g) ^ TL::swz(t8, tqo))) * 16);
    const uint32_t kr0 = k0 - lds_addr(vt) + lds_addr(rt), kr1 = k1 - lds_addr(vt) + lds_addr(rt);
    auto kread = [&](int ks, int mb) -> bf16x8_t {
      const uint32_t base = ks < VKS ? ((ks & 1) ? k1 : k0) : ((ks & 1) ? kr1 : kr0);
      const uint32_t off = ks < VKS ? ((ks >> 1) * 4 + 2 * mb) * 1024 : (2 * mb) * 1024;
      return *MLA_LDS(const bf16x8_t, (uintptr_t)(base + off));
    };
    f32x4_t s[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    bf16x8_t kr[KR][2];
#pragma unroll
    for (int ks = 0; ks < KR - 1; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) kr[ks][mb] = kread(ks, mb);
    __builtin_amdgcn_sched_barrier(0);
    static_for<G::KS>([&](auto KSI) {
      constexpr int ks = decltype(KSI)::value;
      if (ks + KR - 1 < G::KS) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) kr[(ks + KR - 1) % KR][mb] = kread(ks + KR - 1, mb);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % KR][mb], qf[nb][ks], s[mb][nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });

    // softmax in the log2 domain; lane owns head r16, tokens 16mb + 4g + i.
    // Tokens past the range (only in a range's last tile) score -inf.
    bool need = false;
    float mt[2];
    const bool full = tile_start + kTile <= se;   // the same for the whole wave
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      mt[nb] = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = tile_start + 16 * mb + 4 * g + i;
          const float v = full || tok < se ? s[mb][nb][i] * c2 : -INFINITY;
          s[mb][nb][i] = v;
          mt[nb] = fmaxf(mt[nb], v);
        }
      need |= mt[nb] > m_ref[nb] + kSlack;    // also true while m_ref is unset (-inf)
    }
    if (__builtin_expect(__any(need), 0)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float m = mt[nb];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (m_ref[nb] == -INFINITY) {
          m_ref[nb] = m;                     // first tile of the pass
        } else if (m > m_ref[nb] + kSlack) {
          m_init[nb] = m;                    // not representable in this pass
          *flag = 1;
        }
      }
    }
    bf16x8_t pf[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float ls = 0.0f, lm = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pj = __builtin_amdgcn_exp2f(s[mb][nb][i] - m_ref[nb]);
          const __bf16 pb = (__bf16)pj;
          ls += pj;
          pf[nb][4 * mb + i] = pb;
          lm += (float)pb;
        }
      l_sum[nb] += ls;
      l_mma[nb] += lm;
    }
    // P(k) for the PV wave of this SIMD (read after the next barrier)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) *MLA_LDS(bf16x8_t, pb + nb * 1024 + lane * 16) = pf[nb];
    pv<CA, 0, kVRingA>(acc, vt, pf);
  }

  // O^T += V^T P^T over column blocks CB0 .. CB0+N-1 of one tile; V^T read
  // two column blocks ahead through a 3-slot ring (transpose reads: this
  // lane addresses token 16tb + 4g + (r16 >> 2), bytes [8 (r16 & 3), +8) of
  // a 16-column block)
  template <int N, int CB0, int VR>
  static __device__ __forceinline__ void pv(f32x4_t (&acc)[N][2], const char* vt, const bf16x8_t (&pf)[2]) {
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    const int sg = r16 & 3;
    const int t8 = 4 * (g & 1) + (r16 >> 2), tqo = g >> 1;
    // lane part for column blocks with cb & 3 == j is vb + 32 * j (the chunk
    // index 2j + (sg >> 1) enters the swizzle), so keep the four as one base
    // plus per-j terms
    uint32_t voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      voff[j] = lds_addr(vt) + (uint32_t)(tqo * 1024 + (8 * t8 + ((2 * j + (sg >> 1)) ^ TL::swz(t8, tqo))) * 16 +
                                          (sg & 1) * 8);
    auto vread = [&](int cb) -> bf16x8_t {
      const uint32_t a0 = voff[cb & 3] + (cb >> 2) * 4096;
      const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, (uintptr_t)a0));
      const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, (uintptr_t)(a0 + 2048)));
      return bf16x8_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    };
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t vr[VR];
#pragma unroll
    for (int c = 0; c < VR - 1; ++c)
      if (c < N) vr[c] = vread(CB0 + c);
    __builtin_amdgcn_sched_barrier(0);
    static_for<N>([&](auto CI) {
      constexpr int c = decltype(CI)::value;
      if (c + VR - 1 < N) vr[(c + VR - 1) % VR] = vread(CB0 + c + VR - 1);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[c % VR], pf[nb], acc[c][nb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  template <bool QKW, bool NT>
  static __device__ __forceinline__ void run(const DecodeParams& p, int b, int a, int e, int part, int head0, int hg,
                                             char* smem, int* s_table, int* s_flags) {
    const int hb = head0 + 32 * hg;                // this SIMD's heads hb .. hb+31
    constexpr int NACC = QKW ? CA : CBB;
    constexpr int CB0 = QKW ? 0 : CA;              // first column block this wave accumulates

    // Q^T operand (QK wave): lane = head r16 of block nb, dims 32ks + 8g .. +8
    bf16x8_t qf[2][G::KS];
    if constexpr (QKW) {
      const int lane = lane_now();   // Q's per-lane address terms formed here, per piece
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (long long)b * p.q_sb;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int h = hb + 16 * nb + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
          qf[nb][ks] = *reinterpret_cast<const bf16x8_t*>(qb + (long long)h * p.q_sh + 32 * ks + 8 * (lane >> 4));
      }
      wait_vmcnt<0>();
    }

    f32x4_t acc[NACC][2];
    float m_ref[2], l_sum[2], l_mma[2], m_init[2] = {-INFINITY, -INFINITY};
    const float c2 = p.sm_scale * kLog2e;
    auto reset = [&]() {
#pragma unroll
      for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[c][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        m_ref[nb] = m_init[nb];
        l_sum[nb] = 0.0f;
        l_mma[nb] = 0.0f;
      }
    };
    reset();

    const int bs = p.block_size;
    const int32_t* btab = p.block_table + (long long)b * p.bt_stride;
    // One block-table window at a time.  Softmax reference: each head's is
    // fixed by its first tile of the pass and p = 2^(s - m_ref) is summed
    // unscaled; a later tile more than kSlack above it makes every wave zero
    // its state and rewind to a with the larger reference (each redo raises
    // a reference by more than kSlack, so this ends).
#pragma unroll 1
    for (int sa = a; sa < e;) {
      const int pg0 = sa / bs;
      const long long win_end = (long long)(pg0 + TABLE) * bs;
      int se = e;
      if (win_end < e) se = sa + (int)((win_end - sa) / kTile) * kTile;
      __syncthreads();   // earlier readers of s_table, s_flags and the ring are done
      const int npg = (se - 1) / bs - pg0 + 1;
      for (int i = tid_now(); i < npg; i += NW_ * 64) s_table[i] = btab[pg0 + i];
      if (threadIdx.x == 0) {
        s_flags[0] = 0;
        s_flags[1] = 0;
      }
      __syncthreads();

      const int T = (se - sa + kTile - 1) / kTile;
      // No load of this wave is in flight here.  Saying so to the compiler
      // (it does not see the tile loads, which are inline asm) keeps it from
      // guarding registers that an earlier load wrote with a full vmcnt wait
      // inside the tile loop, which would also drain the tile loads.
      wait_vmcnt<0>();
      if constexpr (!QKW) {
        issue<NT>(p, sa, 0, se, pg0, smem, s_table, hg);
        if (T > 1) issue<NT>(p, sa, 1, se, pg0, smem, s_table, hg);
      }
      bool redo = false;
#pragma unroll 1
      for (int k = 0; k <= T; ++k) {
        if constexpr (!QKW) {
          // tile k landed (tile k+1 may still be in flight)
          if (k + 1 < T) wait_vmcnt<LPW>();
          else wait_vmcnt<0>();
        }
        __syncthreads();
        // a redo flagged while computing tile k-1 is seen by all waves here
        if (k > 0 && s_flags[(k - 1) & 1]) {
          redo = true;
          break;
        }
        if constexpr (QKW) {
          if (k < T)
            qk_tile<kKRing>(qf, acc, m_ref, l_sum, l_mma, m_init, vslot(smem, k), rslot(smem, k), pbuf(smem, k, hg),
                       sa + kTile * k, se, c2, &s_flags[k & 1]);
        } else {
          if (k >= 1) {
            const int lane = lane_now();
            bf16x8_t pf[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              pf[nb] = *MLA_LDS(const bf16x8_t, pbuf(smem, k - 1, hg) + nb * 1024 + lane * 16);
            pv<CBB, CA, kVRingB>(acc, vslot(smem, k - 1), pf);
          }
          // Tile k+2 once this wave's PV is issued: tile k+1 has mostly
          // landed by then, so the issue rarely stalls on a full load queue,
          // and it still has about one and a half intervals to land.  (Issued
          // before the PV, or one instruction at a time spread over the PV,
          // the decode time is the same within noise.)
          if (k + 2 < T) issue<NT>(p, sa, k + 2, se, pg0, smem, s_table, hg);
        }
      }
      wait_vmcnt<0>();     // nothing may still be landing when the ring is reused
      if (redo) {
        reset();
        sa = a;
      } else {
        sa = se;
      }
    }

    // ---- finalize: the QK wave owns the softmax sums; it hands 1 / l to the PV wave
    // (lane_now: the per-lane store addresses are worked out here, not hoisted
    // out of the tile loop into registers the loop then holds or spills)
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    __syncthreads();         // every wave is done with the ring and the P buffers
    float* s_inv = reinterpret_cast<float*>(smem);
    float inv[2];
    if constexpr (QKW) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float l = l_sum[nb], lm = l_mma[nb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        lm += __shfl_xor(lm, 16, 64);
        lm += __shfl_xor(lm, 32, 64);
        inv[nb] = 1.0f / lm;
        if (g == 0) {
          s_inv[hg * 32 + 16 * nb + r16] = inv[nb];
          store_partial_lse(p, b, part, hb + 16 * nb + r16, R, (m_ref[nb] + __builtin_amdgcn_logf(l)) * kLn2);
        }
      }
    }
    __syncthreads();
    if constexpr (!QKW) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) inv[nb] = s_inv[hg * 32 + 16 * nb + r16];
    }
    // one column block at a time, so the products need no more registers
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int h = hb + 16 * nb + r16;
#pragma unroll
      for (int c = 0; c < NACC; ++c) {
        const f32x4_t v = acc[c][nb] * inv[nb];
        if (p.direct) store_partial4<true>(p, b, part, h, R, 16 * (CB0 + c) + 4 * g, v[0], v[1], v[2], v[3]);
        else store_partial4<false>(p, b, part, h, R, 16 * (CB0 + c) + 4 * g, v[0], v[1], v[2], v[3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// The two-role stage 1 of Stage1AB for a 128-head group on an fp8 (E4M3)
// cache.  Tiles keep the fp8 layout of TileLoad8 (value columns as 8-token x
// 128-byte blocks, the 64 rope bytes of a token as half blocks), in a 4-slot
// ring for the value columns and a 3-slot ring for the rope columns.  The
// matrix cores read K and V^T from the fp8 tile and convert them to bf16 in
// registers (exact).  P reaches the PV wave as bf16 plus its bf16 rounding
// remainder, the second operand of a second MFMA per V^T fragment, as in
// Stage1's fp8 path; kv_scale scales the scores and the output.  Same
// accumulation order as Stage1's fp8 path: the same bits.
template <int R, int CA>
struct Stage1AB8 {
  using G = Geo<R>;
  using TL8 = TileLoad8<R, 4>;
  static constexpr int NW_ = 8;
  static constexpr int HPG = 128;
  static constexpr int CB = G::CB;
  static constexpr int CBB = CB - CA;
  static_assert(CA >= 1 && CBB >= 1, "column split");
  static constexpr int FG = R / 128;               // full 128-byte column groups (values)
  static constexpr int LPW = FG + 1;               // load instructions per PV wave per tile
  static constexpr int KP = G::KS / 2;             // QK k-step pairs
  static constexpr int VP = R / 64;                // pairs over the value columns
  static constexpr int VSLOT = FG * 4096;
  static constexpr int RSLOT = 4 * 512;
  static constexpr int NV = 4, NR = 3;
  static constexpr int P_OFF = NV * VSLOT + NR * RSLOT;
  static constexpr int PBUF = 2 * HPG * kTile * 2;  // P and its remainder, bf16
  static constexpr int SMEM = P_OFF + 2 * PBUF;
  static constexpr int TABLE = kTableWindow;
  static_assert(SMEM + TABLE * 4 + 8 <= 160 * 1024, "LDS");

  static __device__ __forceinline__ char* vslot(char* smem, int t) { return smem + (t % NV) * VSLOT; }
  static __device__ __forceinline__ char* rslot(char* smem, int t) { return smem + NV * VSLOT + (t % NR) * RSLOT; }
  // per SIMD: P (2 KB) then its remainder (2 KB)
  static __device__ __forceinline__ char* pbuf(char* smem, int t, int hg) {
    return smem + P_OFF + (t & 1) * PBUF + hg * 4096;
  }

  template <bool NT>
  static __device__ __forceinline__ void issue(const DecodeParams& p, int sa, int t, int se, int pg0, char* smem,
                                               const int* s_table, int hg) {
    const int lane = lane_now();
    const typename TL8::Rows rw = TL8::rows(p, sa + kTile * t, se, pg0, s_table, hg);
    char* vb = vslot(smem, t);
    char* rb = rslot(smem, t);
    static_for<FG>([&](auto K) {
      constexpr int k = decltype(K)::value;
      dma16<128 * k, NT>(rw.full[0], lds_addr(vb) + (4 * k + hg) * 1024);
    });
    if (lane < 32) dma16<0, NT>(rw.rope[0], lds_addr(rb) + hg * 512);
  }

  template <bool NT>
  static __device__ void piece(const DecodeParams& p, int b, int a, int e, int part, int head0,
                               char* smem, int* s_table, int* s_flags) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4) run<true, NT>(p, b, a, e, part, head0, wave, smem, s_table, s_flags);
    else run<false, NT>(p, b, a, e, part, head0, wave - 4, smem, s_table, s_flags);
  }

  // V^T fragments from the fp8 tile: in lane group g, source lane
  // r16 = 2i + hh names the token bound to k-slot i and byte half hh of a
  // 16-column block (8-bit transpose read).  The lane's part of the address
  // is worked out once per tile (base and the token's swizzle key); a column
  // block adds an immediate and one xor.
  struct VLane {
    uint32_t base;   // LDS address of the lane's token row in column group 0, plus its byte half
    int t8v;         // swizzle key of that row
  };
  static __device__ __forceinline__ VLane vlane(const char* vt) {
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    const int i8 = r16 >> 1, hh = r16 & 1;
    const int tok = i8 < 4 ? 4 * g + i8 : 12 + 4 * g + i8;
    const int tqv = tok >> 3, t8v = tok & 7;
    return VLane{lds_addr(vt) + (uint32_t)(tqv * 1024 + 8 * t8v * 16 + 8 * hh), t8v};
  }
  static __device__ __forceinline__ v2i32_t vread8(const VLane& vl, int cb) {
    const uint32_t a = vl.base + (uint32_t)((cb >> 3) * 4096) + (uint32_t)(((cb & 7) ^ vl.t8v) * 16);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32(MLA_LDS(v2i32_t, (uintptr_t)a));
  }

  // O^T += V^T (P + remainder)^T over column blocks CB0 .. CB0+N-1, two
  // column blocks at a time: the four products against P, then the four
  // against its remainder, so that each accumulator's second update is four
  // MFMAs behind its first instead of waiting on it back to back (every
  // accumulator still adds P's term, then the remainder's).  V^T fragments
  // go through a 4-slot ring: the current pair and the next pair in flight.
  template <int N, int CB0>
  static __device__ __forceinline__ void pv(f32x4_t (&acc)[N][2], const char* vt, const bf16x8_t (&pf)[2],
                                            const bf16x8_t (&pl)[2]) {
    const VLane vl = vlane(vt);
    __builtin_amdgcn_sched_barrier(0);
    v2i32_t vw[4];
    vw[0] = vread8(vl, CB0);
    if (N > 1) vw[1] = vread8(vl, CB0 + 1);
    __builtin_amdgcn_sched_barrier(0);
    static_for<(N + 1) / 2>([&](auto CI) {
      constexpr int c = 2 * decltype(CI)::value;
      constexpr bool two = c + 1 < N;
      if (c + 2 < N) vw[(c + 2) % 4] = vread8(vl, CB0 + c + 2);
      if (c + 3 < N) vw[(c + 3) % 4] = vread8(vl, CB0 + c + 3);
      const bf16x8_t vf0 = fp8x8_to_bf16((uint32_t)vw[c % 4][0], (uint32_t)vw[c % 4][1]);
      bf16x8_t vf1 = vf0;
      if constexpr (two) vf1 = fp8x8_to_bf16((uint32_t)vw[(c + 1) % 4][0], (uint32_t)vw[(c + 1) % 4][1]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0, pf[nb], acc[c][nb], 0, 0, 0);
      if constexpr (two) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[c + 1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1, pf[nb], acc[c + 1][nb], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[c][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf0, pl[nb], acc[c][nb], 0, 0, 0);
      if constexpr (two) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[c + 1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf1, pl[nb], acc[c + 1][nb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // QK wave, one tile
  static __device__ __forceinline__ void qk_tile(const bf16x8_t (&qf)[2][G::KS], f32x4_t (&acc)[CA][2],
                                                 float (&m_ref)[2], float (&l_sum)[2], float (&l_mma)[2],
                                                 float (&m_init)[2], const char* vt, const char* rt, char* pb,
                                                 int tile_start, int se, float c2, int* flag) {
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    const int t8 = r16 & 7;
    // K fragments straight from the fp8 tile: for k-step pair kp and token
    // block mb, lane (token r16, group g) reads the 16 bytes of dims
    // 64kp + 16g .. +16 and converts them to the bf16 fragments of k-steps
    // 2kp and 2kp + 1 (Q's fragments are loaded in the same order)
    // the lane's part of the K addresses, once per tile: value rows of the
    // two k-step parities (the block and token-block parts are immediates)
    // and the rope row
    const uint32_t kv0 = lds_addr(vt) + (uint32_t)((r16 >> 3) * 1024 + (8 * t8 + (g ^ t8)) * 16);
    const uint32_t kv1 = lds_addr(vt) + (uint32_t)((r16 >> 3) * 1024 + (8 * t8 + ((4 + g) ^ t8)) * 16);
    const uint32_t krp = lds_addr(rt) + (uint32_t)((r16 >> 3) * 512 + (4 * t8 + ((g + (t8 >> 1)) & 3)) * 16);
    auto kread = [&](int kp, int mb) -> u32x4_t {
      const uint32_t ad = kp < VP ? ((kp & 1) ? kv1 : kv0) + (uint32_t)((4 * (kp >> 1) + 2 * mb) * 1024)
                                  : krp + (uint32_t)(2 * mb * 512);
      return *MLA_LDS(const u32x4_t, (uintptr_t)ad);
    };
    f32x4_t s[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) s[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t kw[2][2];
    kw[0][0] = kread(0, 0);
    kw[0][1] = kread(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    // Wave priority: this wave's QK first, then the value wave's products
    // (priority 1, set in run) ahead of this wave's softmax, whose vector
    // work then runs beside them.  Measured (interleaved, same bits):
    // 1524 against 1584 us on the fp8 workload; the same ordering on the
    // bf16 kernel gains nothing there.
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int kp = 0; kp < KP; ++kp) {
      if (kp + 1 < KP) {
        kw[(kp + 1) & 1][0] = kread(kp + 1, 0);
        kw[(kp + 1) & 1][1] = kread(kp + 1, 1);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const u32x4_t w = kw[kp & 1][mb];
        const bf16x8_t k0 = fp8x8_to_bf16(w[0], w[1]);
        const bf16x8_t k1 = fp8x8_to_bf16(w[2], w[3]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[nb][2 * kp], s[mb][nb], 0, 0, 0);
          s[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[nb][2 * kp + 1], s[mb][nb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_setprio(0);
    bool need = false;
    float mt[2];
    // scores scaled to the log2 domain; in a range's last tile the tokens
    // past it score -inf (a uniform branch: full tiles skip the masks)
    auto scale = [&](auto masked) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        mt[nb] = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = tile_start + 16 * mb + 4 * g + i;
            const float v = !decltype(masked)::value || tok < se ? s[mb][nb][i] * c2 : -INFINITY;
            s[mb][nb][i] = v;
            mt[nb] = fmaxf(mt[nb], v);
          }
        need |= mt[nb] > m_ref[nb] + kSlack;
      }
    };
    if (tile_start + kTile <= se) scale(std::false_type{});
    else scale(std::true_type{});
    if (__builtin_expect(__any(need), 0)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float m = mt[nb];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (m_ref[nb] == -INFINITY) {
          m_ref[nb] = m;
        } else if (m > m_ref[nb] + kSlack) {
          m_init[nb] = m;
          *flag = 1;
        }
      }
    }
    // P in bf16 and its bf16 rounding remainder (the value columns are then
    // summed against p to ~16 significant bits)
    bf16x8_t pf[2], pl[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float ls = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pj = __builtin_amdgcn_exp2f(s[mb][nb][i] - m_ref[nb]);
          const __bf16 pb = (__bf16)pj;
          ls += pj;
          pf[nb][4 * mb + i] = pb;
          pl[nb][4 * mb + i] = (__bf16)(pj - (float)pb);
        }
      // P + remainder is within 2^-17 of p: the exact sum normalises acc too
      l_sum[nb] += ls;
      l_mma[nb] += ls;
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      *MLA_LDS(bf16x8_t, pb + nb * 1024 + lane * 16) = pf[nb];
      *MLA_LDS(bf16x8_t, pb + 2048 + nb * 1024 + lane * 16) = pl[nb];
    }
    pv<CA, 0>(acc, vt, pf, pl);
  }

  template <bool QKW, bool NT>
  static __device__ __forceinline__ void run(const DecodeParams& p, int b, int a, int e, int part, int head0, int hg,
                                             char* smem, int* s_table, int* s_flags) {
    const int hb = head0 + 32 * hg;
    constexpr int NACC = QKW ? CA : CBB;
    constexpr int CB0 = QKW ? 0 : CA;
    const float kvs = *p.kv_scale;

    // Q^T operand (QK wave), in the fp8 path's order: k-step pair kp = ks / 2
    // covers dims 64kp .. +64, of which lane group g takes 64kp + 16g .. +16,
    // half ks % 2 in k-step ks
    bf16x8_t qf[2][G::KS];
    if constexpr (QKW) {
      const int lane = lane_now();   // Q's per-lane address terms formed here, per piece
      const int g = lane >> 4;
      const uint16_t* qb = reinterpret_cast<const uint16_t*>(p.q) + (long long)b * p.q_sb;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int h = hb + 16 * nb + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks)
          qf[nb][ks] = *reinterpret_cast<const bf16x8_t*>(qb + (long long)h * p.q_sh + 64 * (ks >> 1) + 16 * g +
                                                          8 * (ks & 1));
      }
      wait_vmcnt<0>();
    }

    f32x4_t acc[NACC][2];
    float m_ref[2], l_sum[2], l_mma[2], m_init[2] = {-INFINITY, -INFINITY};
    const float c2 = p.sm_scale * kvs * kLog2e;
    auto reset = [&]() {
#pragma unroll
      for (int c = 0; c < NACC; ++c)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[c][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        m_ref[nb] = m_init[nb];
        l_sum[nb] = 0.0f;
        l_mma[nb] = 0.0f;
      }
    };
    reset();

    const int bs = p.block_size;
    const int32_t* btab = p.block_table + (long long)b * p.bt_stride;
#pragma unroll 1
    for (int sa = a; sa < e;) {
      const int pg0 = sa / bs;
      const long long win_end = (long long)(pg0 + TABLE) * bs;
      int se = e;
      if (win_end < e) se = sa + (int)((win_end - sa) / kTile) * kTile;
      __syncthreads();
      const int npg = (se - 1) / bs - pg0 + 1;
      for (int i = tid_now(); i < npg; i += NW_ * 64) s_table[i] = btab[pg0 + i];
      if (threadIdx.x == 0) {
        s_flags[0] = 0;
        s_flags[1] = 0;
      }
      __syncthreads();

      const int T = (se - sa + kTile - 1) / kTile;
      wait_vmcnt<0>();   // see Stage1AB: no load of this wave is in flight here
      if constexpr (!QKW) {
        __builtin_amdgcn_s_setprio(1);   // see qk_tile
        issue<NT>(p, sa, 0, se, pg0, smem, s_table, hg);
        if (T > 1) issue<NT>(p, sa, 1, se, pg0, smem, s_table, hg);
      }
      bool redo = false;
#pragma unroll 1
      for (int k = 0; k <= T; ++k) {
        if constexpr (!QKW) {
          if (k + 1 < T) wait_vmcnt<LPW>();
          else wait_vmcnt<0>();
        }
        __syncthreads();
        if (k > 0 && s_flags[(k - 1) & 1]) {
          redo = true;
          break;
        }
        if constexpr (QKW) {
          if (k < T)
            qk_tile(qf, acc, m_ref, l_sum, l_mma, m_init, vslot(smem, k), rslot(smem, k), pbuf(smem, k, hg),
                    sa + kTile * k, se, c2, &s_flags[k & 1]);
        } else {
          if (k >= 1) {
            const int lane = lane_now();
            bf16x8_t pf[2], pl[2];
            const char* pbk = pbuf(smem, k - 1, hg);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              pf[nb] = *MLA_LDS(const bf16x8_t, pbk + nb * 1024 + lane * 16);
              pl[nb] = *MLA_LDS(const bf16x8_t, pbk + 2048 + nb * 1024 + lane * 16);
            }
            pv<CBB, CA>(acc, vslot(smem, k - 1), pf, pl);
          }
          if (k + 2 < T) issue<NT>(p, sa, k + 2, se, pg0, smem, s_table, hg);
        }
      }
      wait_vmcnt<0>();
      if (redo) {
        reset();
        sa = a;
      } else {
        sa = se;
      }
    }

    const int lane = lane_now();   // see Stage1AB: store addresses worked out after the tile loop
    const int g = lane >> 4, r16 = lane & 15;
    __syncthreads();
    float* s_inv = reinterpret_cast<float*>(smem);
    float inv[2];
    if constexpr (QKW) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float l = l_sum[nb], lm = l_mma[nb];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        lm += __shfl_xor(lm, 16, 64);
        lm += __shfl_xor(lm, 32, 64);
        inv[nb] = kvs / lm;
        if (g == 0) {
          s_inv[hg * 32 + 16 * nb + r16] = inv[nb];
          store_partial_lse(p, b, part, hb + 16 * nb + r16, R, (m_ref[nb] + __builtin_amdgcn_logf(l)) * kLn2);
        }
      }
    }
    __syncthreads();
    if constexpr (!QKW) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) inv[nb] = s_inv[hg * 32 + 16 * nb + r16];
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int h = hb + 16 * nb + r16;
#pragma unroll
      for (int c = 0; c < NACC; ++c) {
        const f32x4_t v = acc[c][nb] * inv[nb];
        if (p.direct) store_partial4<true>(p, b, part, h, R, 16 * (CB0 + c) + 4 * g, v[0], v[1], v[2], v[3]);
        else store_partial4<false>(p, b, part, h, R, 16 * (CB0 + c) + 4 * g, v[0], v[1], v[2], v[3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// Token-split stage 1 for one group of 16 * NB heads (bf16 cache).  When
// the token ranges are few (the partial-slot cap binds, or the literal
// partition has fewer items than CUs), a workgroup whose waves share each
// tile would leave each busy CU with a single load stream.  Here four waves
// share the range's heads: wave w streams tiles w, w+4, ... into its own LDS
// slot (its own 32-token tile, loaded by its own instructions and waited on
// by itself alone; the next tile is loaded into the slot group by group as
// the current one's QK and PV finish reading each part, and QK waits for
// each group just before reading it), with its own Q copy, accumulators and softmax
// reference (set by its first tile; a later tile more than kSlack above it
// makes the workgroup redo the range with the larger reference, as in the
// shared-tile kernel, so the accumulators are never rescaled and stay in
// the accumulation registers).  At the end the four partial states are
// merged through LDS, 16 heads at a time, into the range's one partial --
// the same quantity the other kernels store.
template <int R, int NB>
struct Stage1TS {
  using G = Geo<R>;
  using TL = TileLoad<R, 1>;
  static_assert(NB == 1 || NB == 2, "16 or 32 heads");
  static constexpr int NW_ = 4;
  static constexpr int HPG = 16 * NB;
  static constexpr int SLOT = G::TILE_BYTES;
  static constexpr int SMEM = 4 * SLOT;
  static constexpr int TABLE = kTableWindow;
  static constexpr int MERGE_STAT = 4 * 16 * R;     // floats: per-wave accumulators of 16 heads, then statistics
  static constexpr int CQ = G::CHUNKS / 8;          // 1 KB column groups per token quarter: CQ-1 value groups, the rope
  static_assert(TL::LPW == 4 * CQ, "one wave loads the whole tile, 4 token quarters per group");
  static_assert((MERGE_STAT + 4 * 3 * 16) * 4 <= SMEM, "merge area inside the tile slots");

  template <bool NT>
  static __device__ void piece(const DecodeParams& p, int b, int a, int e, int part, int head0,
                               char* smem, int* s_table, int* s_flags) {
    const int lane = lane_now();   // per-lane terms formed per piece, not at kernel entry
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int r16 = lane & 15;

    bf16x8_t qf[NB][G::KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint16_t* qb =
          reinterpret_cast<const uint16_t*>(p.q) + (long long)b * p.q_sb + (long long)(head0 + 16 * nb + r16) * p.q_sh;
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) qf[nb][ks] = *reinterpret_cast<const bf16x8_t*>(qb + 32 * ks + 8 * g);
    }
    // Q is waited for after the window's block table is staged (in flight together)

    uint32_t k_off[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int t8 = r16 & 7, tqo = r16 >> 3, c8 = 4 * par + g;
      k_off[par] = (uint32_t)(tqo * 1024 + (8 * t8 + (c8 ^ TL::swz(t8, tqo))) * 16);
    }
    uint32_t v_off[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sg = r16 & 3;
      const int t8 = 4 * (g & 1) + (r16 >> 2), tqo = g >> 1;
      const int c8 = 2 * k + (sg >> 1);
      v_off[k] = (uint32_t)(tqo * 1024 + (8 * t8 + (c8 ^ TL::swz(t8, tqo))) * 16 + (sg & 1) * 8);
    }

    f32x4_t acc[G::CB][NB];
    float m_ref[NB], l_sum[NB], l_mma[NB], m_init[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) m_init[nb] = -INFINITY;
    const float c2 = p.sm_scale * kLog2e;
    const int bs = p.block_size;
    const int32_t* btab = p.block_table + (long long)b * p.bt_stride;
    char* slot = smem + wave * SLOT;

    // One pass over the range per softmax reference; the redo flag of pass
    // k is s_flags[k & 1] (the other one is cleared for the next pass while
    // no wave can touch it).
    if (threadIdx.x == 0) s_flags[0] = 0;
#pragma unroll 1
    for (int pass = 0;; ++pass) {
#pragma unroll
    for (int cb = 0; cb < G::CB; ++cb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[cb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_ref[nb] = m_init[nb];
      l_sum[nb] = 0.0f;
      l_mma[nb] = 0.0f;
    }
    bool over = false;
    for (int sa = a; sa < e;) {
      const int pg0 = sa / bs;
      const long long win_end = (long long)(pg0 + kTableWindow) * bs;
      int se = e;
      if (win_end < e) se = sa + (int)((win_end - sa) / kTile) * kTile;
      __syncthreads();   // every wave is done with the previous window's table and its slot
      const int npg = (se - 1) / bs - pg0 + 1;
      for (int i = tid_now(); i < npg; i += 4 * 64) s_table[i] = btab[pg0 + i];
      // Q and the table have landed, and no load of this wave is in flight:
      // the tile loop's waits below count this wave's tile loads alone
      wait_vmcnt<0>();
      __syncthreads();
      const int ntiles = (se - sa + kTile - 1) / kTile;
      char* rbuf = slot + (CQ - 1) * 4096;
#pragma unroll 1
      for (int t = wave; t < ntiles; t += 4) {
        const int tile_start = sa + kTile * t;
        // A wave's first tile of the window is issued here; each later one was
        // issued group by group while the previous tile's PV freed its slot.
        // Either way the groups go out rope first, then value groups 0, 1, ...
        // (4 loads each), so QK waits for the group it reads next alone.
        if (t == wave) {
          const typename TL::Rows rw = TL::rows(p, tile_start, se, pg0, s_table, 0);
          static_for<TL::LPW>([&](auto i) {
            TL::template issue<(decltype(i)::value + 4 * (CQ - 1)) % TL::LPW, NT>(rw, slot, rbuf, 0);
          });
        }
        const char* tile = slot;

        f32x4_t sc[2][NB];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) sc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        bf16x8_t kr[3][2];
        wait_vmcnt<4 * (CQ - 2)>();   // the rope and value group 0 have landed
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            kr[ks][mb] = *MLA_LDS(const bf16x8_t, tile + ((ks >> 1) * 4 + 2 * mb) * 1024 + k_off[ks & 1]);
        __builtin_amdgcn_sched_barrier(0);
        static_for<G::KS>([&](auto KSI) {
          constexpr int ks = decltype(KSI)::value;
          if constexpr (ks + 2 < G::KS) {
            // value group (ks + 2) / 2 is read from here on: wait for its 4 loads
            constexpr int gq = (ks + 2) >> 1;
            if constexpr (((ks + 2) & 1) == 0 && gq < CQ - 1) wait_vmcnt<4 * (CQ - 2 - gq)>();
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              kr[(ks + 2) % 3][mb] =
                  *MLA_LDS(const bf16x8_t, tile + (((ks + 2) >> 1) * 4 + 2 * mb) * 1024 + k_off[ks & 1]);
          }
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              sc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % 3][mb], qf[nb][ks], sc[mb][nb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        });

        // The K reads are done (the matrix cores hold them): the rope part of
        // the slot is free, and value group c is free once PV has read it.
        // The wave's next tile goes into those parts as they free up.
        const bool more = t + 4 < ntiles;
        typename TL::Rows nrw;
        if (more) {
          nrw = TL::rows(p, tile_start + 4 * kTile, se, pg0, s_table, 0);
          static_for<4>([&](auto i) { TL::template issue<4 * (CQ - 1) + decltype(i)::value, NT>(nrw, slot, rbuf, 0); });
        }

        // online softmax in the log2 domain; lane owns head 16nb + r16, tokens 16mb + 4g + i
        bf16x8_t pf[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          float mt = -INFINITY;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tok = tile_start + 16 * mb + 4 * g + i;
              const float v = tok < se ? sc[mb][nb][i] * c2 : -INFINITY;
              sc[mb][nb][i] = v;
              mt = fmaxf(mt, v);
            }
          if (__builtin_expect(__any(mt > m_ref[nb] + kSlack), 0)) {   // also true while m_ref is unset
            mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
            mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
            if (m_ref[nb] == -INFINITY) {
              m_ref[nb] = mt;                        // this wave's first tile of the pass
            } else if (mt > m_ref[nb] + kSlack) {
              m_init[nb] = mt;                       // not representable in this pass
              over = true;
            }
          }
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pj = __builtin_amdgcn_exp2f(sc[mb][nb][i] - m_ref[nb]);
              const __bf16 pb = (__bf16)pj;
              l_sum[nb] += pj;
              l_mma[nb] += (float)pb;
              pf[nb][4 * mb + i] = pb;
            }
        }

        auto vread = [&](int cb) -> bf16x8_t {
          const char* vb = tile + (cb >> 2) * 4096 + v_off[cb & 3];
          const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, vb));
          const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(MLA_LDS(bf16x4_t, vb + 2048));
          return bf16x8_t{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        };
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t vr[3];
        vr[0] = vread(0);
        vr[1] = vread(1);
        __builtin_amdgcn_sched_barrier(0);
        static_for<G::CB>([&](auto CBI) {
          constexpr int cb = decltype(CBI)::value;
          if constexpr (cb + 2 < G::CB) vr[(cb + 2) % 3] = vread(cb + 2);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[cb % 3], pf[nb], acc[cb][nb], 0, 0, 0);
          if constexpr ((cb & 3) == 3) {
            // the last read of value group cb / 4 is consumed: refill it
            if (more)
              static_for<4>([&](auto i) { TL::template issue<4 * (cb >> 2) + decltype(i)::value, NT>(nrw, slot, rbuf, 0); });
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      wait_vmcnt<0>();   // (nothing is in flight: a window's last tile issues no successor)
      sa = se;
    }
    if (over) s_flags[pass & 1] = 1;
    __syncthreads();   // every wave's flag is in
    const bool redo = s_flags[pass & 1] != 0;
    if (threadIdx.x == 0) s_flags[(pass + 1) & 1] = 0;
    if (!redo) break;
    }

    // ---- merge the four waves' states into the range's partial, 16 heads at a time
    {
    // the lane is read again so that the merge and store addresses are worked
    // out here, not hoisted into registers the tile loop holds or spills
    const int lane = lane_now();
    const int g = lane >> 4, r16 = lane & 15;
    float* mrg = reinterpret_cast<float*>(smem);
    float* stat = mrg + MERGE_STAT;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float ls = l_sum[nb], lm = l_mma[nb];
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      lm += __shfl_xor(lm, 16, 64);
      lm += __shfl_xor(lm, 32, 64);
      __syncthreads();   // every wave is done with its tile slot (or with the previous 16 heads' merge)
#pragma unroll
      for (int cb = 0; cb < G::CB; ++cb)
        *MLA_LDS(f32x4_t, mrg + ((wave * G::CB + cb) * 64 + lane) * 4) = acc[cb][nb];
      if (g == 0) {
        stat[(wave * 3 + 0) * 16 + r16] = m_ref[nb];
        stat[(wave * 3 + 1) * 16 + r16] = ls;
        stat[(wave * 3 + 2) * 16 + r16] = lm;
      }
      __syncthreads();
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, stat[(w * 3) * 16 + r16]);
      float wt[4], Ls = 0.0f, Lm = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = stat[(w * 3) * 16 + r16];
        wt[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);   // a wave without tiles adds nothing
        Ls += wt[w] * stat[(w * 3 + 1) * 16 + r16];
        Lm += wt[w] * stat[(w * 3 + 2) * 16 + r16];
      }
      const float inv = 1.0f / Lm;
      const int h = head0 + 16 * nb + r16;
      constexpr int CPW = G::CB / 4;   // column blocks each wave writes
      auto out = [&](auto direct) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const int cb = wave * CPW + j;
          f32x4_t o = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < 4; ++w) o += wt[w] * *MLA_LDS(const f32x4_t, mrg + ((w * G::CB + cb) * 64 + lane) * 4);
          const f32x4_t v = o * inv;
          store_partial4<decltype(direct)::value>(p, b, part, h, R, 16 * cb + 4 * g, v[0], v[1], v[2], v[3]);
        }
      };
      if (p.direct) out(std::true_type{});
      else out(std::false_type{});
      if (wave == 0 && g == 0) store_partial_lse(p, b, part, h, R, (M + __builtin_amdgcn_logf(Ls)) * kLn2);
    }
    }
    __syncthreads();   // the merge area is tile slots again for the next piece
  }
};

// Workgroup id -> (work item, head group).  The dispatcher sends id i to XCD
// i % 8; consecutive items (neighbouring token ranges, which share requests,
// their queries and block-table rows) are kept on one XCD, and the head
// groups of one item (which share every KV tile) are dispatched together on
// that XCD, so the shared data meets in its L2.
__device__ __forceinline__ bool map_block(int id, int items, int groups, int& item, int& hg) {
  const int per_xcd = (items + kXcds - 1) / kXcds;
  const int x = id % kXcds;
  const int j = id / kXcds;
  hg = j % groups;
  item = x * per_xcd + j / groups;
  return item < items;
}

__host__ __device__ inline int mapped_grid(int items, int groups) {
  return ((items + kXcds - 1) / kXcds) * kXcds * groups;
}

// Inclusive prefix sum across the wave, 32-bit.  The lane index is read
// through lane_now() so that its derived shuffle indices are not hoisted and
// kept live around the caller's loops.
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  const int ln = lane_now();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = (uint32_t)__builtin_amdgcn_ds_bpermute((ln - o) << 2, (int)v);
    if (ln >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ long long uniform64(long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

template <class K, bool NT>
__global__ __launch_bounds__(K::NW_ * 64) void stage1_mfma_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[K::SMEM];
  __shared__ int s_table[K::TABLE];
  __shared__ int s_flags[2];
  const int groups = p.H / K::HPG;

  // Enumerate this workgroup's pieces (request, token range, partial index)
  // and run each; piece() is inlined at one call site only.  Between pieces
  // only wave-uniform values (scalar registers) and two values per lane stay
  // live, so the pieces keep the vector registers.
  const bool literal = p.partition == PART_LITERAL;
  int item, hg;
  if (!map_block(blockIdx.x, literal ? p.B * p.S : p.G, groups, item, hg)) return;
  const int head0 = hg * K::HPG;
  long long lo = 0, hi = 0, carry = 0;
  int base = 0;
  unsigned long long mask = 0;
  int d_lane = 0, n_lane = 0;      // per lane of the scanned block: padded start - lo, length
  bool done = false;
  if (literal) {
    lo = item;   // the single (request, split) of this workgroup
  } else {
    const BatchTotals t = batch_totals(p.seq_lens, p.B, lane_now());
    const long long total = uniform64(t.total);
    const long long Q = balanced_chunk(BatchTotals{total, 0}, p.G);
    lo = (long long)item * Q;
    hi = min(lo + Q, total);
    done = lo >= hi;
    base = -kWave;
  }
  while (!done) {
    int b, a, e, part;
    if (literal) {
      done = true;
      b = item / p.S;
      const int s = item - b * p.S;
      part = item;                         // slot b * S + s
      const int n = p.seq_lens[b];
      literal_piece_range(n, p.S, p.piece_len, s, a, e);
      if (n <= 0 && p.direct && p.len_min <= 0) {
        // an empty request has no piece: o = 0 and lse = -inf are written
        // here when there is no stage 2 to write them
        constexpr int R = K::G::D - 64;
        uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.o) + ((long long)b * p.H + head0) * R);
        for (int i = tid_now(); i < K::HPG * R / 8; i += K::NW_ * 64) o[i] = make_uint4(0, 0, 0, 0);
        for (int i = tid_now(); i < K::HPG; i += K::NW_ * 64) p.lse[(long long)b * p.H + head0 + i] = -INFINITY;
      }
      if (n <= 0 || e <= a || n < p.len_min || n >= p.len_max) break;
    } else {
      while (mask == 0) {
        base += kWave;
        if (base >= p.B || carry >= hi) break;
        const int bb = base + lane_now();
        const int n = bb < p.B ? max(p.seq_lens[bb], 0) : 0;
        const uint32_t u = (uint32_t)((n + 31) >> 5);          // padded length in 32-token units
        const uint32_t incl = wave_scan_u32(u);
        const long long st = carry + 32LL * (long long)(incl - u);
        mask = __ballot(n > 0 && st < hi && st + n > lo);
        d_lane = (int)(st - lo);                               // used only where the mask is set
        n_lane = n;
        carry += 32LL * (long long)__builtin_amdgcn_readlane(incl, kWave - 1);
      }
      if (mask == 0) break;
      const int j = __ffsll((long long)mask) - 1;
      mask &= mask - 1;
      const int d = __builtin_amdgcn_readlane(d_lane, j);
      const int nn = __builtin_amdgcn_readlane(n_lane, j);
      b = base + j;
      a = d < 0 ? -d : 0;
      e = min((int)(hi - lo) - d, nn);
      part = item + b;                     // slot of the piece (chunk item, request b)
    }
    // the piece is the same for every lane: say so, so that its bounds and
    // loop counters live in scalar registers
    K::template piece<NT>(p, __builtin_amdgcn_readfirstlane(b), __builtin_amdgcn_readfirstlane(a),
             __builtin_amdgcn_readfirstlane(e), __builtin_amdgcn_readfirstlane(part),
             __builtin_amdgcn_readfirstlane(head0), smem, s_table, s_flags);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool mfma_supported(int H, int R, int cache_dtype) {
  return (cache_dtype == DT_BF16 || cache_dtype == DT_FP8) && (R == 512 || R == 256) && H % 16 == 0;
}

bool mfma_group_ok(int hpg) { return hpg == 16 || hpg == 32 || hpg == 64 || hpg == 128; }

// Heads per workgroup: one workgroup takes up to 128 heads (4 waves of 32)
// and reads each tile once; the smaller groups exist for head counts that
// 128 does not divide.  With the literal partition the work items are fixed
// (one per request and split), so when they are too few to fill the GPU the
// heads are split further: the largest group whose workgroups fill every
// resident slot, else 16 (e.g. batch-invariant decode, one item per request).
int mfma_heads_per_group(int H, int R, int cache_dtype, long long literal_items, int cus, int lds_per_cu) {
  int best = H % 128 == 0 ? 128 : H % 64 == 0 ? 64 : H % 32 == 0 ? 32 : 16;
  if (literal_items <= 0) return best;
  for (int hpg = best; hpg >= 16; hpg /= 2) {
    if (H % hpg != 0) continue;
    const long long wgs = literal_items * (H / hpg);
    if (wgs >= (long long)cus * mfma_wgs_per_cu(hpg, R, cache_dtype, lds_per_cu)) return hpg;
  }
  return 16;
}

// Pipeline depth.  A one-wave workgroup (16 or 32 heads) keeps two tiles in
// its ring, so that several such workgroups share a CU (their waves land on
// different SIMDs and hide each other's load stalls); wider workgroups take
// the deepest ring whose wait count fits the 6-bit vmcnt field.
template <int R, int NW, bool F8>
constexpr int stages_for() {
  constexpr int lpw = F8 ? TileLoad8<R, NW>::LPW : Geo<R>::NBLK / NW;
  if constexpr (NW == 1 && !F8) return 2;
  return (2 * lpw < 64) ? 4 : 3;
}

template <class K>
constexpr int lds_bytes() { return K::SMEM + K::TABLE * (int)sizeof(int) + 2 * (int)sizeof(int); }

// the 128-head kernel for an R = 512 bf16 cache, and its column split
template <int R, bool F8>
struct Wide {
  using K = typename std::conditional<
      R == 512,
      typename std::conditional<F8, Stage1AB8<R, 5>, Stage1AB<R, 5, 2, 2, 2>>::type,
      Stage1<R, 2, 4, stages_for<R, 4, F8>(), F8>>::type;
};

template <int R, bool F8>
static int lds_bytes_r(int hpg) {
  switch (hpg) {
    case 128: return lds_bytes<typename Wide<R, F8>::K>();
    case 64: return lds_bytes<Stage1<R, 2, 2, stages_for<R, 2, F8>(), F8>>();
    case 32: return lds_bytes<Stage1<R, 2, 1, stages_for<R, 1, F8>(), F8>>();
    default: return lds_bytes<Stage1<R, 1, 1, stages_for<R, 1, F8>(), F8>>();
  }
}

// Workgroups of a head-group size that fit one CU at once: LDS-bound, and at
// most one wave per SIMD (each wave takes the whole register file share).
int mfma_wgs_per_cu(int hpg, int R, int cache_dtype, int lds_per_cu) {
  const bool f8 = cache_dtype == DT_FP8;
  const int lds = R == 512 ? (f8 ? lds_bytes_r<512, true>(hpg) : lds_bytes_r<512, false>(hpg))
                           : (f8 ? lds_bytes_r<256, true>(hpg) : lds_bytes_r<256, false>(hpg));
  const int waves = hpg >= 128 ? 4 : hpg == 64 ? 2 : 1;   // SIMDs a workgroup's waves occupy
  int n = lds_per_cu / lds;
  if (n > 4 / waves) n = 4 / waves;
  return n < 1 ? 1 : n;
}

template <class K>
static hipError_t launch_k(const DecodeParams& p, hipStream_t stream) {
  const int groups = (p.H + K::HPG - 1) / K::HPG;
  const int items = p.partition == PART_LITERAL ? p.B * p.S : p.G;
  dim3 grid((unsigned)mapped_grid(items, groups)), block(K::NW_ * 64);
  if (p.kv_nt)
    hipLaunchKernelGGL((stage1_mfma_kernel<K, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((stage1_mfma_kernel<K, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int R, bool F8>
static hipError_t launch_r(const DecodeParams& p, hipStream_t stream) {
  switch (p.heads_per_group) {
    case 128: return launch_k<typename Wide<R, F8>::K>(p, stream);
    case 64: return launch_k<Stage1<R, 2, 2, stages_for<R, 2, F8>(), F8>>(p, stream);
    case 32:
      if constexpr (!F8)
        if (p.token_split) return launch_k<Stage1TS<R, 2>>(p, stream);
      return launch_k<Stage1<R, 2, 1, stages_for<R, 1, F8>(), F8>>(p, stream);
    case 16:
      if constexpr (!F8)
        if (p.token_split) return launch_k<Stage1TS<R, 1>>(p, stream);
      return launch_k<Stage1<R, 1, 1, stages_for<R, 1, F8>(), F8>>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stage1_mfma(int cache_dtype, int R, const DecodeParams& p, hipStream_t stream) {
  if (cache_dtype == DT_BF16) return R == 512 ? launch_r<512, false>(p, stream) : launch_r<256, false>(p, stream);
  if (cache_dtype == DT_FP8) return R == 512 ? launch_r<512, true>(p, stream) : launch_r<256, true>(p, stream);
  return hipErrorNotSupported;
}

}  // namespace mla
