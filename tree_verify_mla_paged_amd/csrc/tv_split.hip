// Tree-masked verify attention over a paged MLA latent KV pool: the split
// attention kernel for gfx950.
//
// Computation (page 3 "The Pivot to Live Cutover", sections "The Technical
// Investigation" and "Input Knowledge Required"; page 2 "Flipping the Switch",
// section "The Long Road to Parity"): for every draft row (token t, head h) of
// request b, softmax over the visible gathered latent rows of sm_scale * q.k
// (576 dims), applied to the first 512 dims of those rows, plus the natural
// log-sum-exp.  Visibility is one mask byte per (draft, key), row stride L_b,
// packed beforehand into one 32-bit word per (draft, 32-key tile).
//
// Method: KV-split flash decoding with an LSE merge (page 2, section "The
// Broader Context").  One workgroup per (request, 128-row block, KV split);
// with more than one split it writes a partial output (fp16 under a power-of-
// two scale, or fp32 in precise mode) and its LSE, which tv_merge_kernel
// combines.
//
// gfx950 mapping
//  * 4 wave64s; wave w owns 32 query rows (rows of a request are (draft, head)
//    pairs, head fastest).  All 128 rows share each 32-key tile in LDS.
//  * Tiles are gathered by direct-to-LDS 16-byte loads (global_load_lds_dwordx4):
//    one instruction moves the 1024 bytes of a key's latent dims 0..511, one more
//    per wave moves the 64 RoPE dims of 8 keys, one moves the visibility words.
//    No registers hold in-flight tile data; three LDS stages keep two tiles in
//    flight.  The gathers are inline asm tracked with explicit vmcnt waits, so
//    the compiler sees no aliasing between them and the LDS reads.
//  * S^T[key, row] = K[key, :] . Q[row, :] with v_mfma_f32_32x32x16_bf16:
//    A = key rows read from LDS (ds_read_b128), B = the wave's query rows held
//    in VGPRs for the whole split.  In the 32x32 accumulator layout lane l holds
//    row l % 32 and 16 of the 32 keys: the row max is a 16-register reduction
//    plus one exchange with lane l ^ 32 (v_permlane32_swap).
//  * O^T[d, row] += V^T[d, key] . P^T[key, row] is split by value dims instead:
//    wave w owns dims 128w..128w+127 of all 128 rows (16 accumulators, the 256
//    AGPRs), so the V tile is read once per workgroup rather than once per
//    wave.  The bf16 probabilities go through an LDS buffer in exactly the
//    MFMA B operand layout; A = V^T read straight from the row-major tile with
//    ds_read_b64_tr_b16 (within 16 lanes, output lane i element j comes from
//    source lane 4j + i/4, element i%4: when source lane 4j+q points at dims
//    d0+4q.. of key j, lane i gets keys j=0..3 at dim d0+i).
//  * Software pipeline, one barrier per tile (run_split): the QK chain of tile
//    t+1 carries the gathers of tile t+2 in its shadow, the PV of tile t carries
//    the softmax of tile t+1, a few fenced instructions after each MFMA (one
//    wave per SIMD issues about one instruction every four cycles, so only a
//    handful fit beside each MFMA for free).
//  * Reference maximum with thresholded rescaling: a row's reference is set at
//    the maximum of its first tile with a visible key (O and l are still
//    exactly 0 then) and moves only when a score exceeds it by more than TAU
//    (log2 units).  Probabilities exp2(x - ref) may grow to 2^TAU, which fp32
//    sums and bf16 operands hold, so in the common case no VALU work touches
//    the accumulators.  When a row's reference moves, its l and O are scaled by
//    2^(old - new): the factors go through LDS (every wave holds a slice of
//    every row's O), and each wave rescales, in place in the AGPRs, only the
//    32-row blocks that hold a moved row.
//  * Prologue and epilogue run once per workgroup: accumulators are zeroed by
//    MFMAs; the epilogue stages O through LDS in two buffers and stores rows
//    as contiguous runs.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv_kernels.h"

namespace tv {


constexpr int TILE = TILE_KEYS;
constexpr int ROW = 1088;                 // LDS row pitch of a key's latent dims 0..511
constexpr int MAIN_BYTES = 34816;         // 32 rows at ROW plus the largest key_shift, 256-aligned
constexpr int ROPE_BYTES = TILE * 128;    // RoPE dims 512..575 of 32 keys
constexpr int MASKW_BYTES = 4 * 64 * 4;   // 256 visibility words (one per draft)
constexpr int STAGE = MAIN_BYTES + ROPE_BYTES + MASKW_BYTES;  // 39936
constexpr int NSTAGE = 3;
constexpr int DMA_PER_TILE = 10;          // direct-to-LDS loads per wave per tile
constexpr int SLOT_RING = 4;              // tiles of gather slots held per wave in LDS
constexpr int GM_WIDE = 1;  // gather modes: 64-bit gather addresses
constexpr int GM_NT = 2;    // non-temporal key row loads
constexpr float TAU = 64.0f;              // log2 headroom of a probability over its reference

// A key's 1024 latent bytes sit at key*ROW + key_shift(key).  Modulo 256 bytes
// (one pass over the banks) that is 64*(key & 3) + 16*((key >> 2) & 3): the 16
// keys of a QK read (same chunk) land on 16 distinct 16-byte bank groups, and
// the 4 keys of a transposed PV read (32 contiguous bytes each) on distinct
// groups.  The shift is additive, so every read is a per-lane base plus an
// immediate.
__host__ __device__ constexpr int key_shift(int key) { return 16 * ((key >> 2) & 3); }
static_assert(ROW % 256 == 64, "bank residues assume ROW = 64 mod 256");
static_assert(31 * ROW + key_shift(31) + 1024 <= MAIN_BYTES && MAIN_BYTES % 256 == 0, "");
// XOR swizzle of the 8 RoPE chunks inside a key's 128-byte RoPE row.
__device__ __forceinline__ int rope_swz(int key) { return (key >> 1) & 7; }

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// ---------------------------------------------------------------- split kernel

// Mask bytes of one tile for one wave (byte mode): 2 loads, 4 draft tokens.
constexpr int MASK_J = 2;
static_assert(2 * MASK_J == MASK_BYTES_DRAFTS, "");
struct MaskBytes {
  uint32_t b[MASK_J];
};

// Everything a workgroup needs to gather and consume tiles of its KV split.
struct SplitCtx {
  const uint16_t* kv;
  const int32_t* idx;       // kv_indices of the request
  const uint32_t* wbase;    // visibility words of the block's first draft, split's first tile
  uint32_t wvoff;           // this lane's draft row offset (bytes) from wbase
  uint32_t voff;            // lane * 16: this lane's 16-byte chunk of a latent row
  uint32_t rowb;            // 1152 (bytes per pool row) in a VGPR, the gathers' v_mad operand
  uint32_t rp_voff;         // RoPE gather: this lane's 16-byte RoPE chunk within a pool row
  uint32_t m_main, m_rope, m_mask;  // this wave's gather targets within a stage (bytes)
  int kbeg, kend, ntiles;   // key range [kbeg, kend) of the split, its 32-key tiles
  // contiguous-prefix form: keys below plen are pool slots run0 + key (no
  // index read); plen = 0 otherwise
  int run0, plen;
  int wave, lane;
  // per-lane LDS offsets (relative to a stage)
  int qk_off, pv_off, mw_off;
  int rp_off[4];
  uint32_t al_off;          // this lane's row in a rescale-factor buffer (bytes)
  bool row_ok;
  uint32_t rowm;            // row_ok as a mask: all ones or 0
  float scale_log2;
  lds_u8* sring;            // this wave's ring of gather slots: SLOT_RING entries of 256 bytes
  // Visibility straight from the mask bytes (mbytes: the wave's rows span at
  // most 2 * MASK_J draft tokens): the request's mask at key kbeg of its draft
  // 0 and the bytes of the buffer from there (0 without byte mode); this
  // lane's offset for byte load 0 (draft first + lane / 32, key lane % 32)
  // and the step between loads (2 drafts); for the draft of the lane's row,
  // d = draft - first: the load holding it (dpair = d / 2) and the ballot half
  // (dhalf = 32 * (d % 2)).  Otherwise the words of tv_pack_mask_kernel,
  // gathered with the tile (wbase / wvoff).
  const uint8_t* mrow;
  int mrec;
  uint32_t mvoff, mstep;
  uint32_t dhalf;
  bool dpair;
  bool mbytes;
};

// Direct-to-LDS gathers, as inline asm: the compiler treats the equivalent
// builtin as an access that may complete out of order with LDS reads and then
// waits for all outstanding LDS reads (lgkmcnt(0)) wherever it needs any.
// Their completion is tracked explicitly with vmcnt instead (nothing else in
// the tile loop is a vector memory op).  M0 holds the LDS address; the global
// address is an SGPR base plus a 32-bit VGPR offset, or a 64-bit VGPR address.
// The instruction between the M0 write and the load is the one wait state that
// write needs.
// NT: the key rows are loaded non-temporal (a streaming hint): plans whose
// tiles are read by one workgroup each (one row block) take them once per call,
// and the hint keeps them from displacing what the caches already hold, dirty
// lines included, whose write-back would otherwise share the call's memory
// bandwidth.  Plans of several row blocks leave it off: their row blocks read
// each tile in turn from the L2, and back-to-back calls reuse the
// memory-side cache.
template <bool NT>
__device__ __forceinline__ void dma16_v(const void* vaddr, uint32_t m0) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(vaddr), "s"(m0)
                 : "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(vaddr), "s"(m0)
                 : "m0");
}
__device__ __forceinline__ void dma4_s(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "m0");
}
template <bool NT>
__device__ __forceinline__ void dma16_m0(uint32_t voff, const void* sbase, uint32_t m0) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "m0");
}
// Pool row gathers of a pool under 4 GiB in three instructions: M0 = stage
// target + OFF, byte offset = slot * 1152 + lane chunk (v_mad_u32_u24: slots
// stay below 2^24 there), 16 bytes per lane.  The slot is wave-uniform (SGPR,
// a key's latent row) or per lane (VGPR, the RoPE chunks of 8 keys).
template <int OFF, bool NT>
__device__ __forceinline__ void dma_row_s(uint32_t mb, int slot, const SplitCtx& c) {
  uint32_t a;
  if constexpr (NT)
    asm volatile(
        "s_add_u32 m0, %1, %2\n\t"
        "v_mad_u32_u24 %0, %3, %4, %5\n\t"
        "global_load_lds_dwordx4 %0, %6 nt"
        : "=&v"(a)
        : "s"(mb), "n"(OFF), "s"(slot), "v"(c.rowb), "v"(c.voff), "s"(c.kv)
        : "m0", "scc");
  else
    asm volatile(
        "s_add_u32 m0, %1, %2\n\t"
        "v_mad_u32_u24 %0, %3, %4, %5\n\t"
        "global_load_lds_dwordx4 %0, %6"
        : "=&v"(a)
        : "s"(mb), "n"(OFF), "s"(slot), "v"(c.rowb), "v"(c.voff), "s"(c.kv)
        : "m0", "scc");
}
template <bool NT>
__device__ __forceinline__ void dma_row_v(uint32_t mb, int slot, uint32_t vo, const SplitCtx& c) {
  uint32_t a;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_mad_u32_u24 %0, %2, %3, %4\n\t"
        "global_load_lds_dwordx4 %0, %5 nt"
        : "=&v"(a)
        : "s"(mb), "v"(slot), "v"(c.rowb), "v"(vo), "s"(c.kv)
        : "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_mad_u32_u24 %0, %2, %3, %4\n\t"
        "global_load_lds_dwordx4 %0, %5"
        : "=&v"(a)
        : "s"(mb), "v"(slot), "v"(c.rowb), "v"(vo), "s"(c.kv)
        : "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// A loop-invariant per-lane offset, made opaque so it is recomputed where it is
// used: hoisted out of the tile loop, each (offset + constant) would occupy a
// register of its own instead of folding the constant into the instruction.
__device__ __forceinline__ int fresh(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Register fence: as far as the compiler knows `v` is redefined here, so work
// reading it stays below this point and work producing it stays above.  The
// software pipeline places its steps between chosen MFMAs this way: each step
// fences its inputs where it starts and its outputs where it ends.
template <typename T>
__device__ __forceinline__ void fence(T& v) {
  asm volatile("" : "+v"(v));
}

// Slots of this wave's 8 keys of tile t, gathered into ring entry t % SLOT_RING
// by one direct-to-LDS dword load (lane l: key 8*wave + (l & 7)), clamped to
// the split's last key: keys past the split gather real, finite rows, which are
// masked off and contribute exactly 0.  In the loop it is issued three tiles
// ahead, before the gathers of an earlier tile, so the vmcnt wait that makes
// that tile readable also covers it, and the slots are then plain LDS reads: no
// scalar load is ever pending in the tile loop (a pending one would turn every
// LDS wait into a full wait).  CONTIG: a lane whose key lies in the prefix run
// stores run0 + key into its ring word instead (an LDS store, in order with the
// wave's later ring reads); only draft keys are loaded, so a tile inside the
// prefix issues no load at all.
template <bool CONTIG>
__device__ __forceinline__ void slot_dma(const SplitCtx& c, int t) {
  const int k = min(c.kbeg + t * TILE + 8 * c.wave + (fresh(c.lane) & 7), c.kend - 1);
  if constexpr (CONTIG) {
    if (k < c.plen) {
      *reinterpret_cast<__attribute__((address_space(3))) int*>(
          c.sring + 256 * (t % SLOT_RING) + 4 * c.lane) = c.run0 + k;
    } else {
      dma4_s((uint32_t)k * 4u, c.idx, lds_addr(c.sring) + 256 * (t % SLOT_RING));
    }
  } else {
    dma4_s((uint32_t)k * 4u, c.idx, lds_addr(c.sring) + 256 * (t % SLOT_RING));
  }
}

// The 8 slots of a tile as wave-uniform values, and the slot of key 8*wave +
// lane/8 (the RoPE gather's) per lane: the LDS reads (slot_load), then the
// moves to scalar registers (slot_take, half the slots per call).
typedef int i32x4 __attribute__((ext_vector_type(4)));
struct SlotRaw {
  i32x4 a, b;
  int slane;
};
__device__ __forceinline__ void slot_load(SlotRaw& r, const SplitCtx& c, int t) {
  const lds_u8* e = c.sring + 256 * (t % SLOT_RING);
  r.slane = *reinterpret_cast<const __attribute__((address_space(3))) int*>(
      e + 4 * (fresh(c.lane) >> 3));
  r.a = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(e);
  r.b = *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>(e + 16);
}
__device__ __forceinline__ void slot_take(int (&slot)[8], SlotRaw& r, int half) {
  i32x4& v = half ? r.b : r.a;
  fence(v);
  slot[4 * half + 0] = __builtin_amdgcn_readfirstlane(v[0]);
  slot[4 * half + 1] = __builtin_amdgcn_readfirstlane(v[1]);
  slot[4 * half + 2] = __builtin_amdgcn_readfirstlane(v[2]);
  slot[4 * half + 3] = __builtin_amdgcn_readfirstlane(v[3]);
}

// LDS targets of one stage's gathers for this wave (scalar registers).
struct GatherDst {
  uint32_t main, rope, mask;
};
__device__ __forceinline__ GatherDst gather_dst(const lds_u8* sb, const SplitCtx& c) {
  const uint32_t a = lds_addr(sb);
  return GatherDst{a + c.m_main, a + c.m_rope, a + c.m_mask};
}

// The DMA_PER_TILE direct-to-LDS gathers of one tile, one piece at a time.
//   piece 0..7: latent dims 0..511 of key 8*wave + j, to stage + (8*wave + j)*ROW
//               + key_shift(8*wave + j) = main + j*ROW + 16*(j >> 2);
//   piece 8:    RoPE dims of the wave's 8 keys (one slot per 8 lanes);
//   piece 9:    the visibility words of the tile (one per draft row), unless
//               the mask bytes are read directly (mask_load).
// GM, the gather mode: bit 0 (GM_WIDE) the pool may exceed 4 GiB, so the
// gathers use 64-bit addresses; bit 1 (GM_NT) the key rows are non-temporal
// loads (dma16_v).  The slots are taken by reference to the caller's array (a
// pointer kept in a struct makes the compiler move the array to memory).
template <int GM, int J>
__device__ __forceinline__ void gather_piece(const GatherDst& g, const int (&slot)[8], int slane,
                                             const SplitCtx& c, int t) {
  constexpr bool WIDE = (GM & GM_WIDE) != 0, NT = (GM & GM_NT) != 0;
  if constexpr (J < 8) {
    constexpr int OFF = J * ROW + 16 * (J >> 2);
    if constexpr (WIDE) dma16_m0<NT>(c.voff, c.kv + (int64_t)slot[J] * QK, g.main + OFF);
    else dma_row_s<OFF, NT>(g.main, slot[J], c);
  } else if constexpr (J == 8) {
    if constexpr (WIDE) {
      dma16_v<NT>(reinterpret_cast<const uint8_t*>(c.kv) + (int64_t)slane * (QK * 2) + c.rp_voff,
                  g.rope);
    } else {
      dma_row_v<NT>(g.rope, slane, c.rp_voff, c);
    }
  } else {
    if (!c.mbytes) dma4_s(c.wvoff, c.wbase + min(t, c.ntiles - 1), g.mask);
  }
}

template <int GM>
__device__ __forceinline__ void issue_tile(const lds_u8* sb, const int (&slot)[8], int slane,
                                           const SplitCtx& c, int t) {
  static_assert(DMA_PER_TILE == 10, "");
  const GatherDst g = gather_dst(sb, c);
  gather_piece<GM, 0>(g, slot, slane, c, t);
  gather_piece<GM, 1>(g, slot, slane, c, t);
  gather_piece<GM, 2>(g, slot, slane, c, t);
  gather_piece<GM, 3>(g, slot, slane, c, t);
  gather_piece<GM, 4>(g, slot, slane, c, t);
  gather_piece<GM, 5>(g, slot, slane, c, t);
  gather_piece<GM, 6>(g, slot, slane, c, t);
  gather_piece<GM, 7>(g, slot, slane, c, t);
  gather_piece<GM, 8>(g, slot, slane, c, t);
  gather_piece<GM, 9>(g, slot, slane, c, t);
}

// The MFMAs of the tile loop are inline asm: S^T accumulates in VGPRs and O^T
// in the 256 AGPRs, which the compiler's own allocation does not achieve (it
// puts both in AGPRs and evicts an O block), and `volatile` keeps the LDS
// operand reads issued ahead of them where the source puts them.  Hazards the
// compiler cannot see are covered here: in the tile loop every MFMA operand
// comes from an LDS read or the loop-invariant query registers (never from a
// VALU write just before), the two places where VALU writes feed MFMAs
// (zero_acc, the O rescale) end with s_nop, and results are waited out
// (mfma_drain) before anything but another MFMA reads them.  (One issue slot
// per instruction is what a single wave per SIMD gets: the loop avoids any
// instruction it does not need.)
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// >= 19 wait states: a 16-pass MFMA result may be read by VALU / v_accvgpr_read
__device__ __forceinline__ void mfma_drain_v(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

typedef const __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int PBUF_LO = 4 * 2 * 64 * 16;  // bytes of P^T operands per tile (hi; lo follows)
constexpr int QK_AHEAD = 4;  // LDS operand reads in flight ahead of the QK MFMA chain

// S^T tile (32 keys x this wave's 32 rows) over all 576 dims: A = key rows
// from LDS, B = the wave's query rows, all 36 k-steps held in VGPRs.
__device__ __forceinline__ f32x16 qk_tile(const lds_u8* sb, const bf16x8 (&qf)[QK / 16],
                                          const SplitCtx& c) {
  constexpr int NK = QK / 16;  // 36 k-steps: 32 latent, 4 RoPE
  const lds_u8* qa = sb + c.qk_off;
  auto a_addr = [&](int ks) -> const lds_u8* {
    return ks < VD / 16 ? qa + 32 * ks : sb + c.rp_off[ks - VD / 16];
  };
  bf16x8 buf[QK_AHEAD];
#pragma unroll
  for (int k = 0; k < QK_AHEAD; ++k) buf[k] = *reinterpret_cast<lds_bf16x8*>(a_addr(k));
  f32x16 acc;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const bf16x8 a = buf[ks % QK_AHEAD];
    if (ks + QK_AHEAD < NK)
      buf[ks % QK_AHEAD] = *reinterpret_cast<lds_bf16x8*>(a_addr(ks + QK_AHEAD));
    if (ks == 0) mfma_first_v(acc, a, qf[ks]);
    else mfma_acc_v(acc, a, qf[ks]);
  }
  mfma_drain_v(acc);
  return acc;
}

// Visibility of the lane's row over tile t (bit k = key kbeg + 32*t + k): the
// keys of the split only, nothing for a row past the request.
__device__ __forceinline__ uint32_t tile_valid(const SplitCtx& c, int t);
__device__ __forceinline__ uint32_t mask_finish(uint32_t w, const SplitCtx& c, int t) {
  return w & tile_valid(c, t) & c.rowm;
}
// The lane's gathered word of tile t, unfinished (word mode).
__device__ __forceinline__ uint32_t tile_word(const lds_u8* sb, const SplitCtx& c) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(sb + c.mw_off);
}

// The mask bytes one wave needs for a tile: load j holds key lane % 32 of
// draft first + 2j + lane / 32 (per lane, 0 = hidden).  They are read through a
// buffer resource whose record count ends at the mask's last byte (0 records
// without byte mode), so lanes past the request's drafts or keys read another
// request's bytes or zeros (out of range), never outside the mask; their bits
// are never used.  The loads and ballots are unconditional: a load under a
// branch makes the compiler merge its result with the old value by a copy,
// which waits for every load in flight, the tile gathers included.
__device__ __forceinline__ void mask_load(MaskBytes& m, const SplitCtx& c, int t) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(c.mrow + TILE * t), (short)0, max(c.mrec - TILE * t, 0), 0x00020000);
#pragma unroll
  for (int j = 0; j < MASK_J; ++j)
    m.b[j] = __builtin_amdgcn_raw_buffer_load_b8(r, c.mvoff + j * c.mstep, 0, 0);
}
// The word from the loaded bytes: a ballot per load gives the words of two
// drafts (lanes 0..31, 32..63); each lane shifts its draft's half out of the
// ballot of its pair of drafts.
__device__ __forceinline__ uint32_t mask_word(const MaskBytes& m, const SplitCtx& c, int t) {
  static_assert(MASK_J == 2, "");
  const unsigned long long b0 = __ballot(m.b[0] != 0);
  const unsigned long long b1 = __ballot(m.b[1] != 0);
  const uint32_t x = (uint32_t)(b0 >> c.dhalf), y = (uint32_t)(b1 >> c.dhalf);
  // a row past the request keeps its (clamped) draft's visibility: it writes
  // nothing, and its scores, of zero queries, stay finite
  return (c.dpair ? y : x) & tile_valid(c, t);
}

// QK chain of one tile (as qk_tile) calling bg(ks) after the MFMA of each
// k-step: work that does not depend on the chain, issued in its shadow.  One
// wave per SIMD issues at most one instruction every few cycles, of any kind,
// so only about four fit beside each MFMA for free: bg work is spread thin.
template <typename Bg>
__device__ __forceinline__ f32x16 qk_tile_bg(const lds_u8* sb, const bf16x8 (&qf)[QK / 16],
                                             const SplitCtx& c, Bg&& bg) {
  constexpr int NK = QK / 16;
  const lds_u8* qa = sb + c.qk_off;
  auto a_addr = [&](int ks) -> const lds_u8* {
    return ks < VD / 16 ? qa + 32 * ks : sb + c.rp_off[ks - VD / 16];
  };
  bf16x8 buf[QK_AHEAD];
#pragma unroll
  for (int k = 0; k < QK_AHEAD; ++k) buf[k] = *reinterpret_cast<lds_bf16x8*>(a_addr(k));
  f32x16 acc;
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) {
    const bf16x8 a = buf[ks % QK_AHEAD];
    if (ks + QK_AHEAD < NK)
      buf[ks % QK_AHEAD] = *reinterpret_cast<lds_bf16x8*>(a_addr(ks + QK_AHEAD));
    // one LDS wait per two k-steps: the next step's operand is waited for now
    if ((ks & 1) == 0 && ks + 1 < NK) fence(buf[(ks + 1) % QK_AHEAD]);
    if (ks == 0) mfma_first_v(acc, a, qf[ks]);
    else mfma_acc_v(acc, a, qf[ks]);
    bg(ks);
  }
  mfma_drain_v(acc);
  return acc;
}

// The softmax of one tile, in steps of a few instructions placed between PV
// MFMAs.  S holds S^T of the wave's 32 rows (lane l: row l%32; register i: key
// 8*(i/4) + 4*(l/32) + i%4) and is masked in place; mw is the row's visibility
// word of the tile.  The probabilities stay in registers until the next tile's
// QK chain writes them to the P buffer.
struct Soft {
  float ma, mb, tmax;    // partial row maxima, the tile's row max (log2 units)
  float ref0, alpha_j;   // reference before the tile, 2^(ref0 - tmax)
  float mu;              // reference of the tile's probabilities
  float y0, y1, e0, e1;  // a probability pair: exponents, then values
  bf16x8 pk[2], pl[2];   // P^T operands of k-steps 0 and 1 (lo: precise mode)
};

// mask, max of keys 0-7, of 8-15, row max, reference x3; the exponents of
// probability pair 0; per pair p = 0..7 its two exponentials (step A), then the
// exponents of pair p+1 followed by pair p's sum and bf16 pack (step B); the P
// write: one step per PV MFMA.  The order inside step B keeps an independent
// instruction between each transcendental and the first instruction reading
// its result, and between each exponent and the exponential reading it: the
// hardware needs one wait state there, and an MFMA written as inline asm does
// not count as one for the compiler, which would pad with s_nop instead.
constexpr int SOFT_PRE = 7;
constexpr int SOFT_STEPS = SOFT_PRE + 1 + 2 * 8 + 1;

// v_max3_f32 as written: the fmaxf library form first quiets each input (an
// extra instruction per value); the scores are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// The maximum of 8 values in one asm block: dependent VALU instructions inside
// a block need no wait states, where the compiler pads between separate
// statements whose operands a VALU instruction just wrote.
__device__ __forceinline__ float max8f(float a0, float a1, float a2, float a3, float a4, float a5,
                                      float a6, float a7) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max_f32 %0, %0, %8"
      : "=&v"(r)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(a4), "v"(a5), "v"(a6), "v"(a7));
  return r;
}
// max(m, |a_i|, |b_i|) over two 4-vectors: absolute values as source modifiers
// (no separate instruction per value), one block as above.
__device__ __forceinline__ float max_abs8(float m, const f32x4& a, const f32x4& b) {
  float r;
  asm("v_max3_f32 %0, %1, |%2|, |%3|\n\t"
      "v_max3_f32 %0, %0, |%4|, |%5|\n\t"
      "v_max3_f32 %0, %0, |%6|, |%7|\n\t"
      "v_max3_f32 %0, %0, |%8|, |%9|"
      : "=&v"(r)
      : "v"(m), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]),
        "v"(b[3]));
  return r;
}

template <bool PRECISE>
__device__ __forceinline__ void write_p(lds_u8* pb, const SplitCtx& c, const Soft& sm);

// A tile's visibility before the choice between its sources, made in the
// softmax's first step: the gathered word unfinished (ww) with the tile's key
// range (valid), or the word from the mask bytes, finished (wb).
struct MaskSel {
  uint32_t ww, wb, valid;
};
__device__ __forceinline__ uint32_t tile_valid(const SplitCtx& c, int t) {
  const int rem = c.kend - (c.kbeg + t * TILE);
  return rem >= TILE ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
}

// alpha_u: the LDS address of the tile's rescale factors; pb_u: its P buffer.
template <bool PRECISE>
__device__ __forceinline__ void soft_step(int step, Soft& sm, f32x16& S, MaskSel& ms,
                                          const SplitCtx& c, float& m_ref, float& l_sum,
                                          uint32_t alpha_u, lds_u8* pb_u) {
  if (step == 0) {
    fence(S);
    fence(ms.ww);
    const uint32_t mw = c.mbytes ? ms.wb : (ms.ww & ms.valid & c.rowm);
    // a tile every row of the wave sees whole (every prefix tile) skips this
    // uniform branch; masked scores are -inf
    if (!__all(mw == 0xffffffffu)) {
      const uint32_t mh = mw >> (4 * (c.lane >> 5));  // constant bit positions below
#pragma unroll
      for (int i = 0; i < 16; ++i)
        S[i] = ((mh >> (8 * (i >> 2) + (i & 3))) & 1u) ? S[i] : -INFINITY;
    }
    fence(S);
  } else if (step == 1 || step == 2) {
    fence(S);
    const int o = 8 * (step - 1);
    const float m = max8f(S[o], S[o + 1], S[o + 2], S[o + 3], S[o + 4], S[o + 5], S[o + 6],
                          S[o + 7]);
    if (step == 1) {
      sm.ma = m;
      fence(sm.ma);
    } else {
      sm.mb = m;
      fence(sm.mb);
    }
  } else if (step == 3) {
    fence(sm.mb);
    const float m = max3f(sm.ma, sm.mb, sm.mb) * c.scale_log2;  // the scale is positive
    // the other half of the row: v_permlane32_swap leaves, in each lane, the
    // other half's value in one of its two results (no LDS round trip)
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                     false, false);
    sm.tmax = max3f(m, __uint_as_float(sw[0]), __uint_as_float(sw[1]));
    fence(sm.tmax);
  } else if (step == 4) {
    // first visible keys set the reference (O and l are still 0)
    fence(sm.tmax);
    sm.ref0 = (m_ref == -INFINITY) ? sm.tmax : m_ref;
    sm.alpha_j = __builtin_amdgcn_exp2f(sm.ref0 - sm.tmax);
    fence(sm.ref0);
    fence(sm.alpha_j);
  } else if (step == 5) {
    // a score more than TAU above the reference moves it, and l and O are
    // scaled by 2^(old - new) (alpha is exactly 1 otherwise)
    fence(sm.alpha_j);
    const bool jump = sm.tmax > sm.ref0 + TAU;
    const float alpha = jump ? sm.alpha_j : 1.f;
    l_sum *= alpha;
    m_ref = jump ? sm.tmax : sm.ref0;
    sm.alpha_j = alpha;
    fence(sm.alpha_j);
    fence(l_sum);
    fence(m_ref);
  } else if (step == 6) {
    fence(sm.alpha_j);
    sm.mu = (m_ref == -INFINITY) ? 0.f : m_ref;
    // both halves of a row write the same factor: no lane masking
    *reinterpret_cast<__attribute__((address_space(3))) float*>(
        (uintptr_t)(alpha_u + c.al_off)) = sm.alpha_j;
    fence(sm.mu);
  } else if (step == SOFT_STEPS - 1) {
    write_p<PRECISE>(pb_u, c, sm);
  } else {
    // probability pairs: keys i, i+1 of pair p = i / 2 (one packed bf16 pair)
    const int j = step - SOFT_PRE;
    const int p = j == 0 ? 0 : (j - 1) / 2;
    const bool step_a = j > 0 && (j - 1) % 2 == 0;
    const int i = 2 * p;
    // the exponents of pair q
    auto exponents = [&](int q) {
      float x0 = S[2 * q], x1 = S[2 * q + 1];
      fence(x0);
      fence(x1);
      sm.y0 = __builtin_fmaf(x0, c.scale_log2, -sm.mu);
      sm.y1 = __builtin_fmaf(x1, c.scale_log2, -sm.mu);
      fence(sm.y0);
      fence(sm.y1);
    };
    if (j == 0) {
      exponents(0);
    } else if (step_a) {
      fence(sm.y1);
      sm.e0 = __builtin_amdgcn_exp2f(sm.y0);
      sm.e1 = __builtin_amdgcn_exp2f(sm.y1);
      fence(sm.e0);
      fence(sm.e1);
    } else {
      if (p + 1 < 8) exponents(p + 1);
      fence(sm.e1);
      l_sum += sm.e0;
      l_sum += sm.e1;
      fence(l_sum);
      bf16x8& hk = sm.pk[i >> 3];
      hk[i & 7] = (__bf16)sm.e0;
      hk[(i & 7) + 1] = (__bf16)sm.e1;
      // PRECISE: the rounding residuals, themselves rounded to bf16 (hi + lo
      // carries about 16 significant bits of a probability)
      if (PRECISE) {
        bf16x8& lk = sm.pl[i >> 3];
        lk[i & 7] = (__bf16)(sm.e0 - (float)hk[i & 7]);
        lk[(i & 7) + 1] = (__bf16)(sm.e1 - (float)hk[(i & 7) + 1]);
        fence(lk);
      }
      fence(hk);
    }
  }
}

// The PV MFMA after which each softmax step runs: one step per MFMA (32 per
// tile), or per second MFMA in precise mode (64).
template <bool PRECISE>
__device__ __forceinline__ constexpr int soft_at(int step) {
  return (PRECISE ? 2 : 1) * step;
}
static_assert(soft_at<false>(SOFT_STEPS - 1) < 32 && soft_at<true>(SOFT_STEPS - 1) < 64, "");

// P^T of this wave's rows into a P buffer: register i of lane l is key
// 8*(i/4) + 4*(l/32) + i%4 of row l%32, which is exactly the B operand layout of
// k-steps 0 (i < 8) and 1.
template <bool PRECISE>
__device__ __forceinline__ void write_p(lds_u8* pb, const SplitCtx& c, const Soft& sm) {
  typedef __attribute__((address_space(3))) bf16x8 lds_w16;
  lds_u8* w = pb + c.wave * 2048 + fresh(c.lane * 16);
  *reinterpret_cast<lds_w16*>(w) = sm.pk[0];
  *reinterpret_cast<lds_w16*>(w + 1024) = sm.pk[1];
  if (PRECISE) {
    *reinterpret_cast<lds_w16*>(w + PBUF_LO) = sm.pl[0];
    *reinterpret_cast<lds_w16*>(w + PBUF_LO + 1024) = sm.pl[1];
  }
}

// gather_piece with the piece number known only after unrolling
template <int GM>
__device__ __forceinline__ void gather_piece_n(int j, const GatherDst& g, const int (&slot)[8],
                                               int slane, const SplitCtx& c, int t) {
  static_assert(DMA_PER_TILE == 10, "");
  switch (j) {
    case 0: gather_piece<GM, 0>(g, slot, slane, c, t); break;
    case 1: gather_piece<GM, 1>(g, slot, slane, c, t); break;
    case 2: gather_piece<GM, 2>(g, slot, slane, c, t); break;
    case 3: gather_piece<GM, 3>(g, slot, slane, c, t); break;
    case 4: gather_piece<GM, 4>(g, slot, slane, c, t); break;
    case 5: gather_piece<GM, 5>(g, slot, slane, c, t); break;
    case 6: gather_piece<GM, 6>(g, slot, slane, c, t); break;
    case 7: gather_piece<GM, 7>(g, slot, slane, c, t); break;
    case 8: gather_piece<GM, 8>(g, slot, slane, c, t); break;
    default: gather_piece<GM, 9>(g, slot, slane, c, t); break;
  }
}

// A operand of PV k-step kst, dim block db: V^T of 8 dims x 16 keys by two
// transposed 8-byte reads (k-step kst covers keys 16*kst + {4*half + 0..3,
// 8 + 4*half + 0..3}).
__device__ __forceinline__ bf16x8 pv_a(const lds_u8* sb, const SplitCtx& c, int kst, int db) {
  const lds_u8* va = sb + c.pv_off;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(va + (16 * kst) * ROW + 64 * db));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(va + (16 * kst + 8) * ROW + 32 + 64 * db));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
}

// The A operands PV reads first (dim block 0; both k-steps, or k-step 0 in
// precise mode): they depend only on the tile, so they are read before the
// barrier that publishes P.
template <bool PRECISE>
__device__ __forceinline__ void pv_a_first(bf16x8 (&A0)[2], const lds_u8* sb, const SplitCtx& c) {
  A0[0] = pv_a(sb, c, 0, 0);
  if (!PRECISE) A0[1] = pv_a(sb, c, 1, 0);
}

// PV of tile t (stage sb), after the barrier that publishes P(t): first the O
// rescale if some row's reference moved in this tile (resc, read ahead from the
// tile's flag; alpha_t: its factors), then the MFMAs, each followed by bg(i)
// (work that does not depend on them, issued in their shadow).  A0: the first
// A operands (pv_a_first).
template <bool PRECISE, typename Bg>
__device__ __forceinline__ void pv_tile(const lds_u8* sb, const SplitCtx& c, const lds_u8* pbuf,
                                        f32x16 (&O)[16], bool resc, const float* alpha_t,
                                        const bf16x8 (&A0)[2], Bg&& bg) {
  if (resc) {
    // some row's reference moved: scale this wave's O slice of the rows, for
    // each 32-row block that holds such a row (accumulator O[4*db + rb] holds
    // rows 32*rb + lane % 32; the branch per block is uniform)
    float a4[4];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) a4[rb] = alpha_t[32 * rb + (c.lane & 31)];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (__any(a4[rb] != 1.f)) {
        // in place in the AGPRs (O must never have a definition outside the
        // accumulator register class in the loop), one asm block per
        // accumulator: read, multiply and write back four elements at a time
        // through four VGPRs.  (One block per element made the compiler pad
        // each with a wait state: a fourth instruction per element.)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          f32x16& o = O[4 * db + rb];
          float t0, t1, t2, t3;
#define TV_RESCALE4(i0, i1, i2, i3)                 \
  "v_accvgpr_read_b32 %16, %" #i0 "\n\t"          \
  "v_accvgpr_read_b32 %17, %" #i1 "\n\t"          \
  "v_accvgpr_read_b32 %18, %" #i2 "\n\t"          \
  "v_accvgpr_read_b32 %19, %" #i3 "\n\t"          \
  "v_mul_f32 %16, %16, %20\n\t"                   \
  "v_mul_f32 %17, %17, %20\n\t"                   \
  "v_mul_f32 %18, %18, %20\n\t"                   \
  "v_mul_f32 %19, %19, %20\n\t"                   \
  "v_accvgpr_write_b32 %" #i0 ", %16\n\t"         \
  "v_accvgpr_write_b32 %" #i1 ", %17\n\t"         \
  "v_accvgpr_write_b32 %" #i2 ", %18\n\t"         \
  "v_accvgpr_write_b32 %" #i3 ", %19\n\t"
          asm volatile(TV_RESCALE4(0, 1, 2, 3) TV_RESCALE4(4, 5, 6, 7)
                       TV_RESCALE4(8, 9, 10, 11) TV_RESCALE4(12, 13, 14, 15)
                       : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]), "+a"(o[4]),
                         "+a"(o[5]), "+a"(o[6]), "+a"(o[7]), "+a"(o[8]), "+a"(o[9]),
                         "+a"(o[10]), "+a"(o[11]), "+a"(o[12]), "+a"(o[13]), "+a"(o[14]),
                         "+a"(o[15]), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
                       : "v"(a4[rb]));
#undef TV_RESCALE4
        }
      }
    }
    asm volatile("s_nop 3");  // accumulator writes before the next MFMA reads them
  }
  // O^T[dims of db, rows of rb] += V^T . P^T: A operand (dim block db of this
  // wave) from pv_a, B operand (row block rb) from the P buffer.
  const lds_u8* pb = pbuf + fresh(c.lane * 16);
  auto pv_b = [&](int kst, int rb) -> bf16x8 {
    return *reinterpret_cast<lds_bf16x8*>(pb + rb * 2048 + kst * 1024);
  };
  if (!PRECISE) {
    // all 8 B operands stay live; the A operands of one dim block (both
    // k-steps) are read while the previous block's 8 MFMAs run
    bf16x8 B[2][4], A[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) B[0][i] = pv_b(0, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) B[1][i] = pv_b(1, i);
    A[0][0] = A0[0];
    A[0][1] = A0[1];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int cur = db & 1;
#pragma unroll
      for (int kst = 0; kst < 2; ++kst) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          mfma_acc_a(O[4 * db + rb], A[cur][kst], B[kst][rb]);
          bg(8 * db + 4 * kst + rb);
        }
        if (db + 1 < 4) A[cur ^ 1][kst] = pv_a(sb, c, kst, db + 1);
      }
    }
  } else {
    // k-step outer: the 4 hi and 4 lo B operands of one k-step stay live, each
    // A operand feeds 8 MFMAs
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      bf16x8 Bh[4], Bl[4], A[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Bh[i] = pv_b(kst, i);
        Bl[i] = *reinterpret_cast<lds_bf16x8*>(pb + PBUF_LO + i * 2048 + kst * 1024);
      }
      A[0] = kst == 0 ? A0[0] : pv_a(sb, c, kst, 0);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        if (db + 1 < 4) A[(db + 1) & 1] = pv_a(sb, c, kst, db + 1);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          mfma_acc_a(O[4 * db + rb], A[db & 1], Bh[rb]);
          bg(32 * kst + 8 * db + rb);
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          mfma_acc_a(O[4 * db + rb], A[db & 1], Bl[rb]);
          bg(32 * kst + 8 * db + 4 + rb);
        }
      }
    }
  }
}

// Start of the split (c.ntiles >= 1), in two parts around the query loads.
// split_slots: the slot loads of tiles 0..2 (nothing outstanding before them).
template <bool CONTIG>
__device__ __forceinline__ void split_slots(const SplitCtx& c) {
  slot_dma<CONTIG>(c, 0);
  slot_dma<CONTIG>(c, 1);
  slot_dma<CONTIG>(c, 2);
}
// split_gathers: once the slots have landed (the caller waits), the gathers of
// tiles 0 and 1 and their mask bytes.
template <int GM>
__device__ __forceinline__ void split_gathers(lds_u8* stages, const SplitCtx& c, MaskBytes& m0,
                                              MaskBytes& m1) {
  int slot[8];
  SlotRaw r;
  slot_load(r, c, 0);
  slot_take(slot, r, 0);
  slot_take(slot, r, 1);
  if (c.mbytes) {
    mask_load(m0, c, 0);
    mask_load(m1, c, 1);  // (past the split: real bytes or zeros, unused)
  }
  issue_tile<GM>(stages, slot, r.slane, c, 0);
  if (c.ntiles > 1) {
    slot_load(r, c, 1);
    slot_take(slot, r, 0);
    slot_take(slot, r, 1);
    issue_tile<GM>(stages + STAGE, slot, r.slane, c, 1);
  }
}

// Whether some row's reference moved in a tile: its rescale factors (alpha_t,
// 128 rows) are not all exactly 1.
__device__ __forceinline__ void alpha_load(float& a0, float& a1, const float* alpha_t,
                                           const SplitCtx& c) {
  a0 = alpha_t[c.lane];
  a1 = alpha_t[c.lane + 64];
}
__device__ __forceinline__ int alpha_moved(float a0, float a1) {
  return __any(a0 != 1.f || a1 != 1.f) ? 1 : 0;
}

// Iteration t's QK chain (tile t+1, stage nx1) with, in its shadow: the read
// of tile t's rescale factors; if GATHER, the slots and gathers of tile t+2
// (stage nx2) and the slots of tile t+3; then tile t+1's visibility words and
// the first PV operands of tile t (stage cur).  Tile t+1's visibility comes
// back as mww (the gathered word, unfinished) and mwb (from the mask bytes: mb
// holds tile t+1's, turned into the word early in the chain, and then receives
// tile t+2's); the softmax's first step picks one (MaskSel), so that nothing
// in the chain waits for the word's LDS read.
template <int GM, bool PRECISE, bool GATHER, bool CONTIG>
__device__ __forceinline__ f32x16 qk_phase(lds_u8* stages, const SplitCtx& c,
                                           const bf16x8 (&qf)[QK / 16], const float* alpha_t,
                                           int t, int cur, int nx1, int nx2, uint32_t& mww,
                                           uint32_t& mwb, int& resc, bf16x8 (&A0)[2],
                                           MaskBytes& mb) {
  constexpr int G0 = 5;  // first gather piece; then one every third k-step
  static_assert(G0 + 3 * (DMA_PER_TILE - 1) + 2 < QK / 16, "");
  SlotRaw r;
  int slot[8];
  float a0, a1;
  const GatherDst g = gather_dst(stages + nx2 * STAGE, c);
  auto bg = [&](int ks) {
    if (ks == 0) {
      if (GATHER) {
        slot_load(r, c, t + 2);
        slot_dma<CONTIG>(c, t + 3);
      }
    } else if (ks == 1) {
      alpha_load(a0, a1, alpha_t, c);
    } else if (ks == 2 || ks == 3) {
      if (GATHER) slot_take(slot, r, ks - 2);
      if (ks == 3 && c.mbytes) {
        mwb = mask_word(mb, c, t + 1);  // tile t+1's bytes
        fence(mwb);  // here, in the chain's shadow, not where it is used
      }
    } else if (ks == 4) {
      fence(a0);
      fence(a1);
      resc = alpha_moved(a0, a1);
    } else if (ks >= G0 && ks < G0 + 3 * DMA_PER_TILE && (ks - G0) % 3 == 0) {
      if (GATHER) gather_piece_n<GM>((ks - G0) / 3, g, slot, r.slane, c, t + 2);
      if (GATHER && ks == G0 + 3 * (DMA_PER_TILE - 1) && c.mbytes) mask_load(mb, c, t + 2);
    } else if (ks == G0 + 3 * DMA_PER_TILE - 2) {
      if (!c.mbytes) mww = tile_word(stages + nx1 * STAGE, c);
    } else if (ks == G0 + 3 * DMA_PER_TILE - 1) {
      pv_a_first<PRECISE>(A0, stages + cur * STAGE, c);
    }
  };
  return qk_tile_bg(stages + nx1 * STAGE, qf, c, bg);
}

// All tiles of the split after split_gathers, software-pipelined, one barrier per
// tile.  Tile k sits in stage k % 3, its P in P buffer k % 2 and its rescale
// factors in alpha_s[k % 2].  Iteration t, after its barrier, runs the QK chain
// of tile t+1 (qk_phase: the gathers of tile t+2 in its shadow), then the PV of
// tile t with, in its shadow, the softmax of tile t+1, which ends by writing
// P(t+1) and tile t+1's factors.  The barrier of iteration t publishes tile
// t+1's gathers (every gather issued before it has landed: vmcnt(0), the
// iteration issues nothing else to global memory), P(t) and tile t's factors,
// and frees stage t-1, P buffer t-1 and factors t-1 for reuse.  The softmax of
// tile 0 runs ahead of the loop.
template <int GM, bool PRECISE, bool CONTIG>
__device__ __forceinline__ void run_split(lds_u8* stages, const SplitCtx& c, lds_u8* pbuf,
                                          bf16x8 (&qf)[QK / 16], f32x16 (&O)[16],
                                          float& m_ref, float& l_sum, float* alpha_s,
                                          const MaskBytes& m0, MaskBytes& mb) {
  constexpr int PB = PRECISE ? 2 * PBUF_LO : PBUF_LO;  // bytes of one P buffer
  const int nt = c.ntiles;
  const uint32_t alpha_lds = lds_addr((lds_u8*)alpha_s);
  // tile 0: its gathers landed, and with them the query loads issued before
  // them (only tile 1's nine row gathers may be outstanding; each load the
  // compiler sees, such as the mask bytes, it waits for itself); QK, softmax
  if (nt > 1) wait_vmcnt<DMA_PER_TILE - 1>();
  else wait_vmcnt<0>();
  __syncthreads();
  Soft sm;
  {
    f32x16 S = qk_tile(stages, qf, c);
    // every query register is known to have landed before the tile loop (an
    // asm use of each makes the compiler wait here at the latest): otherwise
    // it keeps them pending at the loop header and puts a vmcnt wait before
    // each QK MFMA, which in steady state waits out the tile gathers instead
#pragma unroll
    for (int ks = 0; ks < QK / 16; ++ks) asm volatile("" : "+v"(qf[ks]));
    MaskSel ms{0u, 0u, tile_valid(c, 0)};
    if (c.mbytes) ms.wb = mask_word(m0, c, 0);
    else ms.ww = tile_word(stages, c);
#pragma unroll
    for (int st = 0; st < SOFT_STEPS; ++st)
      soft_step<PRECISE>(st, sm, S, ms, c, m_ref, l_sum, alpha_lds, pbuf);
  }
  int cur = 0;  // stage of tile t
  for (int t = 0; t < nt; ++t) {
    const int nx1 = cur == NSTAGE - 1 ? 0 : cur + 1;  // stage of tile t+1
    const int nx2 = cur == 0 ? NSTAGE - 1 : cur - 1;  // stage of tile t+2
    // (unconditional: on the last iteration nothing is in flight, and the
    // compiler then knows every load it issued has landed here)
    wait_vmcnt<0>();
    __syncthreads();
    const float* alpha_t = alpha_s + ROWS_PER_WG * (t & 1);
    f32x16 S;
    // tile t+1's visibility (none past the last tile)
    MaskSel ms{0u, 0u, 0u};
    int resc;         // some row's reference moved in tile t
    bf16x8 A0[2];
    if (t + 2 < nt) {
      S = qk_phase<GM, PRECISE, true, CONTIG>(stages, c, qf, alpha_t, t, cur, nx1, nx2, ms.ww,
                                                ms.wb, resc, A0, mb);
      ms.valid = tile_valid(c, t + 1);
    } else if (t + 1 < nt) {
      S = qk_phase<GM, PRECISE, false, CONTIG>(stages, c, qf, alpha_t, t, cur, nx1, nx2, ms.ww,
                                                 ms.wb, resc, A0, mb);
      ms.valid = tile_valid(c, t + 1);
    } else {
      float a0, a1;
      alpha_load(a0, a1, alpha_t, c);
      pv_a_first<PRECISE>(A0, stages + cur * STAGE, c);
      resc = alpha_moved(a0, a1);
      S = f32x16{};  // a tile past the end: its softmax below masks it off whole
    }
    const uint32_t alpha_n = alpha_lds + 4 * ROWS_PER_WG * ((t + 1) & 1);
    lds_u8* pb_n = pbuf + PB * ((t + 1) & 1);
    pv_tile<PRECISE>(stages + cur * STAGE, c, pbuf + PB * (t & 1), O, resc != 0, alpha_t, A0,
                     [&](int i) {
#pragma unroll
                       for (int st = 0; st < SOFT_STEPS; ++st)
                         if (i == soft_at<PRECISE>(st))
                           soft_step<PRECISE>(st, sm, S, ms, c, m_ref, l_sum, alpha_n, pb_n);
                     });
    cur = nx1;
  }
  // drain: no gather may still be writing LDS when the epilogue reuses it
  wait_vmcnt<0>();
  __syncthreads();
}

// Epilogue helpers.  The staging layout: row r of a wave's region is 512 bytes
// (its 128 dims in fp32), the 16-byte granule g (dims 4g..4g+3 of the slice)
// at slot g ^ r.  The writes go down columns (a write: granules 2j, 2j+1 of
// 32 rows) and the reads along rows (8 lanes a row, every other granule); with
// the XOR both spread over all banks.  A slot address is the lane's base XOR a constant:
// the base holds the row's 512-aligned offset and the lane's own bits of the
// slot, the constant the granule bits the instruction picks.
//
// O^T of row block RB (accumulators O[4*db + RB]) into the staging region:
// this lane's row r, granules 8*db + 2*q + half (dims 32*db + 8*q + 4*half +
// 0..3, the accumulator's elements 4q..4q+3).  `base` = region offset + 512*r
// + 16*(half ^ r).
template <int RB>
__device__ __forceinline__ void stage_rows(lds_u8* buf, uint32_t base, const f32x16 (&O)[16]) {
  // The 16 addresses are formed here, beside the writes (which the LDS write
  // rate bounds), not hoisted ahead of the barrier before the first block.  The
  // writes are asm so that the compiler does not merge the row blocks' copies
  // of this code, which would route the accumulators through VGPRs.
  asm volatile("" : "+v"(base));
  const uint32_t b0 = (uint32_t)(uintptr_t)buf;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x16& o = O[4 * db + RB];
      const f32x4 v = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
      asm volatile("ds_write_b128 %0, %1" : : "v"(b0 + (base ^ (128 * db + 32 * q))), "a"(v) : "memory");
    }
  // the compiler does not count asm LDS writes: it would drop the wait that
  // the barrier after every staging needs
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ f16x8 to_f16x8(const f32x4& a, const f32x4& b) {
  return f16x8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
               (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

// A 16-byte store at device scope (sc1): it is written through this XCD's L2 as
// it happens, instead of staying there dirty until the kernel's end writes the L2
// back; the data still lands in the memory-side cache, where the merge kernel
// reads it.  Used for the fp16 partial outputs, where it was measured: the split
// kernel's end comes 2-3 us sooner at 32 MB of partials, the merge unchanged.
// (For the fp32 partials of precise mode, twice the bytes and stores, it made the
// split kernel 20-40 % slower; those stay ordinary stores.)  A store
// of more than 8 bytes reads its data registers after issue, and a VALU write to
// them needs a wait state in between, which the compiler inserts only for
// stores it can see: the s_nop is that wait.
template <typename T>
__device__ __forceinline__ void store_dev16(void* ptr, const T& v) {
  static_assert(sizeof(T) == 16, "");
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(ptr), "v"(v) : "memory");
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x4& a, const f32x4& b) {
  return bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
}

// O = 0 by MFMAs with zero operands: 16 instructions instead of 256
// accumulator writes (this code, too, runs cold once per workgroup).
__device__ __forceinline__ void zero_acc(f32x16 (&O)[16]) {
  bf16x8 z = bf16x8{};
  asm volatile("s_nop 1" : "+v"(z));  // z was just written by VALU moves
#pragma unroll
  for (int i = 0; i < 16; ++i)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(O[i]) : "v"(z));
}

template <int GM, bool PRECISE, bool MASKB, bool CONTIG>
__global__ __launch_bounds__(256, 1) void tv_split_kernel(
    const uint16_t* __restrict__ q_, const uint16_t* __restrict__ kv_,
    const int32_t* __restrict__ kv_indices_, const int32_t* __restrict__ kv_indptr_,
    const int32_t* __restrict__ qo_indptr_, const uint8_t* __restrict__ mask_,
    const int32_t* __restrict__ mask_indptr_, const uint32_t* __restrict__ mask_words_,
    const int32_t* __restrict__ order_, void* __restrict__ out_, float* __restrict__ lse_,
    void* __restrict__ ws_o_, float* __restrict__ ws_lse_, SplitScalars p) {
  // one LDS block: the tile stages, then the two P buffers (the epilogue's two
  // staging buffers span both), then the slot rings
  constexpr int PB2 = 2 * (PRECISE ? 2 * PBUF_LO : PBUF_LO);
  __shared__ __attribute__((aligned(1024))) uint8_t lds_s[NSTAGE * STAGE + PB2 + 4 * SLOT_RING * 256];
  __shared__ float inv_s[ROWS_PER_WG];
  __shared__ float alpha_s[2 * ROWS_PER_WG];
  lds_u8* const stages = (lds_u8*)lds_s;
  lds_u8* const pbuf = stages + NSTAGE * STAGE;
  lds_u8* const sring_s = pbuf + PB2;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // blockIdx -> dispatch position -> work item.  Dispatch fills the 8 XCDs
  // round-robin by blockIdx; XCD x = blockIdx % 8 takes groups of xcd_group
  // consecutive positions (the row blocks of a KV split share its gathered
  // tiles through that XCD's L2), the groups going round-robin over the XCDs
  // in position order (gridDim.x is a multiple of 8 * xcd_group).  Positions
  // map to work items through the longest-first order when there is one.
  const int G = p.xcd_group;
  const int xk = blockIdx.x >> 3;
  const int pos = (((xk / G) << 3) + (blockIdx.x & 7)) * G + xk % G;
  if (pos >= p.total_work) return;
  const int work = order_ ? order_[pos] : pos;
  if (work < 0) return;
  const int rb = work % p.row_blocks;
  const int s = (work / p.row_blocks) % p.max_splits;
  const int b = work / (p.row_blocks * p.max_splits);

  const int q0 = qo_indptr_[b];
  const int nq = qo_indptr_[b + 1] - q0;
  const int k0 = kv_indptr_[b];
  const int L = kv_indptr_[b + 1] - k0;  // the mask's row stride
  const int H = p.num_heads;
  const int R = nq * H;
  const int row0 = rb * ROWS_PER_WG;
  if (row0 >= R) return;
  // Keys considered: at most the plan's max_tiles * 32, so a request longer
  // than max_kv_len (a broken precondition) still stays inside the plan: with
  // split_keys a multiple of 32 that caps the split count at max_splits (the
  // partial buffers' extent, absent with one split) and the visibility word of
  // every tile inside its row.
  const int Lk = min(L, p.max_tiles * TILE);
  const int nsplit = Lk > 0 ? (Lk + p.split_keys - 1) / p.split_keys : 1;
  if (s >= nsplit) return;

  SplitCtx c;
  c.kv = kv_;
  c.idx = kv_indices_ + k0;
  c.kbeg = s * p.split_keys;
  c.kend = min(Lk, c.kbeg + p.split_keys);
  c.ntiles = c.kend > c.kbeg ? (c.kend - c.kbeg + TILE - 1) / TILE : 0;
  c.wave = wave;
  c.lane = lane;
  c.scale_log2 = p.scale_log2;
  // contiguous-prefix form: the request's first prefix entry names its run
  // (nothing read past it; a request without prefix reads nothing here)
  c.plen = CONTIG ? max(L - nq, 0) : 0;
  c.run0 = (CONTIG && c.plen > 0) ? kv_indices_[k0] : 0;
  c.sring = sring_s + wave * (SLOT_RING * 256);

  const int i0 = row0 / H;
  const int nd = (min(row0 + ROWS_PER_WG, R) - 1) / H - i0 + 1;
  // this lane's query row
  const int r = row0 + wave * 32 + l32;
  c.row_ok = r < R;
  c.rowm = c.row_ok ? 0xffffffffu : 0u;
  const int dl = c.row_ok ? r / H - i0 : 0;
  const int64_t g = (int64_t)q0 * H + r;  // global row = token * H + head
  // visibility words of draft i0 + d, tile 0 of the split: row (q0 + i0 + d)
  c.wbase = mask_words_ + (int64_t)(q0 + i0) * p.max_tiles + c.kbeg / TILE;
  c.wvoff = (uint32_t)min(64 * wave + lane, nd - 1) * (uint32_t)p.max_tiles * 4u;
  c.voff = (uint32_t)lane * 16u;
  asm volatile("v_mov_b32 %0, 0x480" : "=v"(c.rowb));  // QK * 2, kept in a register
  c.rp_voff = VD * 2 + 16 * ((lane & 7) ^ rope_swz(8 * wave + (lane >> 3)));
  c.m_main = 8 * wave * ROW + 32 * (wave & 1);
  c.m_rope = MAIN_BYTES + 8 * wave * 128;
  c.m_mask = MAIN_BYTES + ROPE_BYTES + 256 * wave;
  c.al_off = 4 * (wave * 32 + l32);

  // per-lane LDS read offsets (relative to a stage)
  c.qk_off = l32 * ROW + key_shift(l32) + 16 * half;  // + 32*ks: latent chunk 2*ks + half
#pragma unroll
  for (int j = 0; j < 4; ++j)  // RoPE chunk 2*j + half of key l32
    c.rp_off[j] = MAIN_BYTES + l32 * 128 + 16 * ((2 * j + half) ^ rope_swz(l32));
  // PV transposed reads: 16-lane group g16 = lane >> 4 picks dims +16*(g16 & 1);
  // source lane sl = lane & 15 points at key 4*half + sl/4, dims 4*(sl & 3)..+3.
  // Key 16*kst + 8*rd + 4*half + sl/4, dims 128*wave + 32*db + 16*(g16 & 1) +
  // 4*(sl & 3): pv_off + (16*kst + 8*rd)*ROW + 32*rd + 64*db, since
  // key_shift(key) = 16*(2*rd + half) is additive in rd
  {
    const int sl = lane & 15;
    c.pv_off = (4 * half + (sl >> 2)) * ROW + 16 * half + 256 * wave +
               32 * ((lane >> 4) & 1) + 8 * (sl & 3);
  }
  c.mw_off = MAIN_BYTES + ROPE_BYTES + 4 * dl;
  c.mbytes = MASKB;  // a constant: every branch on it folds
  {
    // the first draft of the wave's rows (a wave past the request's rows: its last)
    const int first = min(row0 + 32 * wave, R - 1) / H;
    const int64_t moff = (int64_t)mask_indptr_[b] + c.kbeg;
    c.mrow = mask_ + moff;
    c.mrec = c.mbytes ? (int)((int64_t)p.total_mask - moff) : 0;
    c.mvoff = (uint32_t)(first + half) * (uint32_t)L + (uint32_t)l32;
    c.mstep = 2u * (uint32_t)L;
    const int d = min(r, R - 1) / H - first;  // < MASK_BYTES_DRAFTS in byte mode
    c.dpair = d >= 2;
    c.dhalf = 32u * (uint32_t)(d & 1);
  }

  // prologue: the slot loads, then the query rows (their transfer overlaps the
  // slots' round trip), then the first two tiles' gathers
  if (c.ntiles > 0) split_slots<CONTIG>(c);

  // query rows -> MFMA B operands (k = dims 16*ks + 8*half .. +7), all 576
  // dims in VGPRs for the whole split.  A row past the request's rows loads
  // nothing (zeros): its scores stay in its own lane, are masked off, and it
  // writes nothing.  A wave issues the QK / 16 loads iff it has a row of the
  // request (uniform: its first row is one).
  bf16x8 qf[QK / 16];
  const bool wave_q = row0 + wave * 32 < R;
#pragma unroll
  for (int ks = 0; ks < QK / 16; ++ks) qf[ks] = bf16x8{};
  MaskBytes m0 = {}, mb = {};  // mask bytes of tiles 0 and 1 (byte mode)
  if (c.ntiles > 0) {
    if (c.row_ok) {
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(q_ + g * QK + half * 8);
#pragma unroll
      for (int ks = 0; ks < QK / 16; ++ks) qf[ks] = qp[2 * ks];
    }
    // the slots have landed once at most the query loads are outstanding
    if (wave_q) wait_vmcnt<QK / 16>();
    else wait_vmcnt<0>();
    split_gathers<GM>(stages, c, m0, mb);
  }

  // O^T of dims 128*wave + 32*db .. +31 (register r of lane l: dim + 8*(r/4) +
  // 4*(l/32) + r%4) and rows 32*rb + l%32: accumulator O[4*db + rb]
  f32x16 O[16];
  zero_acc(O);
  float m_ref = -INFINITY;  // reference maximum (log2 units)
  float l_sum = 0.f;        // this half's share of the normaliser
  if (c.ntiles > 0)
    run_split<GM, PRECISE, CONTIG>(stages, c, pbuf, qf, O, m_ref, l_sum, alpha_s, m0, mb);

  // the last PV MFMAs must finish before O is read out of the AGPRs
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]),
                 "+a"(O[6]), "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]),
                 "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
  const float l_tot = l_sum + __shfl_xor(l_sum, 32);
  const bool empty = !(l_tot > 0.f);
  // v_log_f32 is log2
  const float lse_nat = empty ? -INFINITY
                              : (m_ref + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994530942f;
  if (half == 0) inv_s[wave * 32 + l32] = empty ? 0.f : 1.f / l_tot;
  if (c.row_ok && half == 0) {
    if (nsplit == 1) lse_[g] = lse_nat;
    else if (PRECISE) ws_lse_[g * p.max_splits + s] = lse_nat;
    else ws_lse_[2 * (g * p.max_splits + s)] = lse_nat;  // the scale exponent follows
  }
  __syncthreads();

  // O^T -> LDS -> global, one row block (32 rows) at a time: wave w puts its
  // 128 dims of the 32 rows into region w ([32 rows][512 bytes], granules
  // XOR-swizzled by row as described at stage_rows); then 8 lanes store each
  // row: lane i of a row covers dims 64k + 8i .. +7, k = 0..7, so that each
  // store instruction writes whole contiguous row segments.  Two staging
  // buffers: the row block after the current one is staged while the current
  // one's stores drain.  The row-block loop is rolled (this code runs once per
  // workgroup).
  constexpr int EP_ROW = 512;
  constexpr int EPB = 4 * 32 * EP_ROW;
  static_assert(2 * EPB <= NSTAGE * STAGE + PB2, "");
  {
    const uint32_t wbase = (uint32_t)(wave * 32 * EP_ROW + l32 * EP_ROW + 16 * (half ^ l32));
    const int lr = tid >> 3, si = tid & 7;       // row within the row block, lane in the row
    const int nrb = min(4, (R - row0 + 31) >> 5);  // row blocks holding a row of the request
    stage_rows<0>(stages, wbase, O);
    __syncthreads();
#pragma unroll 1
    for (int rb = 0; rb < nrb; ++rb) {
      // chunk k (dims 64k + 8*si .. +7) is region k/2, granules 16*(k&1) +
      // 2*si + {0, 1} of row lr
      const uint32_t rbase = (uint32_t)((rb & 1) * EPB + lr * EP_ROW + 16 * ((2 * si) ^ lr));
      const int rl = 32 * rb + lr;  // row within the workgroup's block
      f32x4 x[16];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          x[2 * k + h] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
              stages + (rbase ^ (256 * (k & 1) + 16 * h)) + (k >> 1) * 32 * EP_ROW);
      float inv = inv_s[rl];
      const int64_t gr = (int64_t)q0 * H + row0 + rl;
      const bool live = row0 + rl < R;
      if (nsplit > 1 && !PRECISE) {
        // fp16 partial with an exact power-of-two scale per row: with the
        // row's max |o| < 2^e, o * 2^(15 - e) stays below 2^15 (no overflow,
        // values down to 2^-29 of the max stay normal); o = h * 2^(e - 15).
        // The scale folds into the 1/l multiply.
        float m = 0.f, m2 = 0.f;  // two independent chains
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          m = max_abs8(m, x[k], x[k + 1]);
          m2 = max_abs8(m2, x[k + 8], x[k + 9]);
        }
        m = max3f(m, m2, m2);
        float d = dpp_f<0xb1>(m);  // the 8 lanes of the row: pairs, quads, halves of 8
        m = max3f(m, d, d);
        d = dpp_f<0x4e>(m);
        m = max3f(m, d, d);
        d = dpp_f<0x141>(m);
        m = max3f(m, d, d);
        const int e = __builtin_amdgcn_frexp_expf(m * inv);
        inv = __builtin_ldexpf(inv, 15 - e);
        if (live) {
          const int64_t wi = gr * p.max_splits + s;
          _Float16* o = static_cast<_Float16*>(ws_o_) + wi * VD + 8 * si;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            store_dev16(o + 64 * k, to_f16x8(x[2 * k] * inv, x[2 * k + 1] * inv));
          if (si == 0) ws_lse_[2 * wi + 1] = (float)(e - 15);
        }
      } else if (live) {
        if (nsplit > 1 || p.out_f32) {
          float* o = nsplit > 1 ? static_cast<float*>(ws_o_) + (gr * p.max_splits + s) * VD
                                : static_cast<float*>(out_) + gr * VD;
          o += 8 * si;
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            *reinterpret_cast<f32x4*>(o + 64 * k) = x[2 * k] * inv;
            *reinterpret_cast<f32x4*>(o + 64 * k + 4) = x[2 * k + 1] * inv;
          }
        } else {
          __bf16* o = static_cast<__bf16*>(out_) + gr * VD + 8 * si;
#pragma unroll
          for (int k = 0; k < 8; ++k)
            *reinterpret_cast<bf16x8*>(o + 64 * k) = to_bf16x8(x[2 * k] * inv, x[2 * k + 1] * inv);
        }
      }
      // the next row block into the other buffer (last read two blocks ago)
      switch (rb + 1 < nrb ? rb : 3) {
        case 0: stage_rows<1>(stages, wbase + EPB, O); break;
        case 1: stage_rows<2>(stages, wbase, O); break;
        case 2: stage_rows<3>(stages, wbase + EPB, O); break;
        default: break;
      }
      __syncthreads();
    }
  }
}

// Launches go through hipLaunchKernel, which reports this launch's own status
// (a non-gfx950 device fails here: the library carries gfx950 code only).  With
// events, hipExtLaunchKernel stamps them with the dispatch's own start and end
// times: no separate marker packets enter the stream around the kernel.

hipError_t launch_split(const SplitParams& p, int grid, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1) {
  const uint16_t* q = p.q;
  const uint16_t* kv = p.kv;
  const int32_t* kvi = p.kv_indices;
  const int32_t* kvp = p.kv_indptr;
  const int32_t* qop = p.qo_indptr;
  const uint8_t* mk = p.mask;
  const int32_t* mkp = p.mask_indptr;
  const uint32_t* mw = p.mask_words;
  const int32_t* ord = p.order;
  void* o = p.out;
  float* l = p.lse;
  void* wo = p.ws_o;
  float* wl = p.ws_lse;
  SplitScalars sc = p.s;
  void* args[] = {&q, &kv, &kvi, &kvp, &qop, &mk, &mkp, &mw, &ord, &o, &l, &wo, &wl, &sc};
  // [gather mode: wide | non-temporal][precise][mask bytes][contiguous prefix]
#define TV_SPLIT_FN(G, P, M, C) reinterpret_cast<const void*>(&tv_split_kernel<G, P, M, C>)
#define TV_SPLIT_FN2(G, P, M) {TV_SPLIT_FN(G, P, M, false), TV_SPLIT_FN(G, P, M, true)}
#define TV_SPLIT_FN4(G, P) {TV_SPLIT_FN2(G, P, false), TV_SPLIT_FN2(G, P, true)}
#define TV_SPLIT_FN8(G) {TV_SPLIT_FN4(G, false), TV_SPLIT_FN4(G, true)}
  static const void* const fns[4][2][2][2] = {TV_SPLIT_FN8(0), TV_SPLIT_FN8(1), TV_SPLIT_FN8(2),
                                              TV_SPLIT_FN8(3)};
#undef TV_SPLIT_FN8
#undef TV_SPLIT_FN4
#undef TV_SPLIT_FN2
#undef TV_SPLIT_FN
  const int gm = (p.wide ? GM_WIDE : 0) | (p.stream_kv ? GM_NT : 0);
  const void* fn = fns[gm][p.precise][p.s.mask_bytes != 0][p.contig];
  if (ev0 || ev1) return hipExtLaunchKernel(fn, dim3(grid), dim3(256), args, 0, st, ev0, ev1, 0);
  return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, st);
}
}  // namespace tv
