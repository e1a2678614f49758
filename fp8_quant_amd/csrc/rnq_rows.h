// Row kernel: RMSNorm -> partial NeoX RoPE -> (optional) per-row FP8 e4m3fn.
//
// Operation: tilelang-tutorial chapter 13 fusion page, torch_reference_fused
// and the two fused kernels; chapter 28 case study, the QK-norm prologue
// (rows are (token, head) pairs; every head of a token uses the token's
// cos/sin row; one fp32 scale per row).
//
// Mapping (gfx950, wave64).
//  * A row of D = 16*L elements is split into L "units" of two 16-byte chunks,
//    one unit per lane: a rope unit holds chunk j of the lower half of the
//    rope tail and chunk j of the upper half (the lane owns both members of
//    its 8 RoPE pairs, so no exchange is needed); a plain unit holds two
//    adjacent chunks. A wave covers G = 64/L rows per "pass"; each wave-wide
//    load covers whole 128-byte spans of 8 rows (D = 128). The fp8 codes
//    leave as whole 16-byte chunks: two neighbouring rope lanes swap halves
//    (one DPP move per dword) so that each store writes whole lines.
//  * W waves take the passes round-robin (wave w takes w, w + W, w + 2W, ...),
//    so the waves in flight work on one narrow window of the tensors and DRAM
//    pages are used whole. W is about what stays resident, or more for large
//    launches (at most 8 passes per wave; later waves start in launch order as
//    earlier ones retire). Every wave runs the same number of passes; the few
//    slots past the end repeat the final pass, which writes the same bytes
//    again.
//  * Software pipeline: the input chunks of the next NS - 1 passes (with their
//    cos/sin chunks on aligned rope passes) and, on per-lane rows, the cos/sin
//    values of the next pass are in flight while a pass is computed; with
//    positions, the next pass's position comes with its input and its table
//    values go out from the middle of the current pass.
//    No memory access in the steady state is conditional (clamped indices,
//    every lane of a row storing the same scale), so the in-order memory
//    counter can be waited on precisely.
//  * When every pass stays inside one token and one tensor (heads and q heads
//    both multiples of G, the usual QK layout), a pass's token and tensor are
//    wave-uniform and its addresses are one scalar base plus lane-constant
//    offsets. When instead every pass holds whole tokens of one tensor (G a
//    multiple of the heads per token: one row per token of path R, the
//    RMSNorm forward, a single-tensor prologue), the same holds with the
//    pass's first token as the base: the rows of its G / heads tokens sit at
//    lane-constant offsets, their table rows are consecutive, and each rope
//    lane loads its own row's 8 cos and 8 sin values with the pass's input (the
//    rows of such a pass have tokens of their own: nothing to share through
//    LDS). Such launches are short, so the weight, cos, sin and positions
//    pointers ride in preloaded argument slots (RowHot). Otherwise each lane
//    locates its own row.
//  * Inputs may be views: the rows of a token are contiguous in each input
//    tensor, and consecutive tokens are xs0 / xs1 elements apart (q and k
//    inside a fused QKV projection output). Outputs are contiguous.
//  * The cos/sin row of token t is row t, or row positions[t] of a
//    position-indexed table (clamped into it), gathered as it is read.
//  * Each wave stages its own copy of the two weight vectors in LDS (fp32).
//  * Row sums: sum of squares in fp64 (exact for 16-bit inputs) and the
//    absmax, each reduced over the L lanes with DPP.
//  * Workgroups are renumbered so that neighbouring row ranges (which share
//    tokens) run on the same XCD and its L2.
#pragma once

#include <math.h>

#include <type_traits>

#include "rnq_device.h"
#include "rnq_launch.h"

namespace rnq {

constexpr int RW = 4;  // waves per workgroup
constexpr int RT = 64 * RW;

#ifndef RNQ_ROWS_CHUNKED
#define RNQ_ROWS_CHUNKED 0
#endif
#ifndef RNQ_ROWS_STAGES
#define RNQ_ROWS_STAGES 2
#endif
// passes of input in flight per wave plus the one in use, for aligned rope
// passes (table rows through LDS); other modes use two
constexpr int NS_STAGED = RNQ_ROWS_STAGES;
static_assert(NS_STAGED >= 2, "at least the pass in use and the next one");

// Variants of the pass loop chosen once per wave: GEN = per-pass branches for
// fp8_max below 1 or a clamp that can bind; FULL = the rope tail is the whole
// row; XCH = codes stored as whole 16-byte chunks after a swap inside each
// pair of rope lanes (aligned passes whose plain part and rope tail are both
// multiples of 32 columns).
template <bool GEN, bool FULL, bool XCH = false>
struct Opts {
  static constexpr bool gen = GEN, full = FULL, xch = XCH;
};

// Where one lane's row of a pass lives.
struct Loc {
  uint32_t row;   // flattened (token, head) index (clamped into range)
  uint32_t tok;
  uint32_t trow;  // cos/sin table row (the token, or its position)
  uint32_t ri;    // row index inside its tensor
  uint32_t ri0;   // aligned passes: row index of the pass's first row (wave-uniform)
  uint64_t xoff;  // element offset of the input row (aligned passes: of the pass's first row)
  bool second;    // row of tensor 1 (k)
};

// A pass's input chunks (and, on aligned rope passes, this lane's piece of the
// token's cos and sin rows, loaded with them: the first 4, 8 or 16 bytes).
struct Table {
  float4 c0, c1, s0, s1;  // this lane's values (per-lane rows, and passes of whole tokens)
};
struct Data {
  Loc loc;
  uint4 xa, xb;
  uint4 cw, sw;
  Table tab;     // passes of whole tokens: this lane's cos / sin values
  uint32_t pos;  // passes of whole tokens with positions: this lane's token's position
};

// The fields a wave needs before its first input load. They reach the kernel
// as leading scalar arguments (14 dwords), which gfx950 preloads into scalar
// registers at wave launch: the first input loads then go out without
// waiting for a load of the kernel arguments (one memory latency per launch).
// On passes of whole tokens (one tensor) the slots that only the two-tensor
// layout and the head division need carry what such a pass needs before its
// first compute, so that the first pass's weights, positions and table rows go
// out with its input instead of after a load of the kernel arguments:
//   x1_or_mt = w0, xs0 = cos, xs1 = sin, heads | heads0 << 32 = positions,
//   div_magic = the token stride in elements (below 2^30 there), and the token
//   shift (log2 of the rows per token) in div_shift's byte.
struct RowHot {
  const uint16_t* x0;
  uint64_t x1_or_mt;  // x1, or w0 on passes of whole tokens
  uint64_t xs0, xs1;  // token strides, or cos and sin on passes of whole tokens
  uint32_t waves, passes, heads, heads0, div_magic;
  uint32_t shift_rope;  // div_shift (or tok_shift) | rope << 8
  __device__ __forceinline__ uint32_t div_shift() const { return shift_rope & 0xffu; }
  __device__ __forceinline__ uint32_t rope() const { return shift_rope >> 8; }
  __device__ __forceinline__ const uint16_t* x1() const { return (const uint16_t*)x1_or_mt; }
  __device__ __forceinline__ uint32_t tok_shift() const { return shift_rope & 0xffu; }
  __device__ __forceinline__ const uint16_t* mt_w0() const { return (const uint16_t*)x1_or_mt; }
  __device__ __forceinline__ const float* mt_cos() const { return (const float*)xs0; }
  __device__ __forceinline__ const float* mt_sin() const { return (const float*)xs1; }
  __device__ __forceinline__ const int32_t* mt_pos() const {
    return (const int32_t*)((uint64_t)heads0 << 32 | heads);
  }
  __device__ __forceinline__ uint32_t mt_xs() const { return div_magic; }
};

__device__ __forceinline__ uint32_t div_heads(const RowHot& h, uint32_t row) {
  return (uint32_t)(((uint64_t)row * h.div_magic) >> h.div_shift());  // row / heads, exact below 2^31
}

template <int G, int D, bool ALIGNED, bool POS, bool MT>
__device__ __forceinline__ Loc locate(const RowParams& p, const RowHot& hp, uint32_t pass, uint32_t slot) {
  Loc r;
  if constexpr (MT) {
    // whole tokens of tensor 0: the pass's first row and token are wave-uniform
    // (with positions, each lane reads its own token's, see load_input)
    static_assert(ALIGNED, "several tokens per pass: aligned");
    const uint32_t row0 = __builtin_amdgcn_readfirstlane(pass * (uint32_t)G);
    const uint32_t t = __builtin_amdgcn_readfirstlane(row0 >> hp.tok_shift());
    r.second = false;
    r.tok = t;
    r.ri0 = row0;
    r.ri = row0 + slot;
    r.row = row0 + slot;
    r.xoff = (uint64_t)t * hp.mt_xs();
  } else if constexpr (ALIGNED) {
    // the whole pass lies inside one token and one tensor, and the launch
    // holds whole passes only: everything but the slot is wave-uniform
    // (readfirstlane: keep the wave-uniform values in scalar registers through
    // every control-flow merge, so descriptors built from them stay scalar)
    const uint32_t row0 = __builtin_amdgcn_readfirstlane(pass * (uint32_t)G);
    const uint32_t t = __builtin_amdgcn_readfirstlane(div_heads(hp, row0));
    const uint32_t h0 = row0 - t * hp.heads;
    r.second = h0 >= hp.heads0;
    const uint32_t hk = __builtin_amdgcn_readfirstlane(r.second ? h0 - hp.heads0 : h0);  // head inside its tensor
    const uint32_t ri0 = __builtin_amdgcn_readfirstlane(r.second ? t * (hp.heads - hp.heads0) + hk : t * hp.heads0 + hk);
    r.tok = t;
    r.ri0 = ri0;
    r.ri = ri0 + slot;
    r.row = row0 + slot;
    r.xoff = (uint64_t)t * (r.second ? hp.xs1 : hp.xs0) + (uint64_t)hk * D;
  } else {
    // rows past the end repeat the last row (same inputs, same bytes written)
    const uint32_t row = min(pass * (uint32_t)G + slot, p.total_rows - 1);
    r.row = row;
    const uint32_t t = div_heads(hp, row);
    const uint32_t h = row - t * hp.heads;
    r.tok = t;
    r.second = h >= hp.heads0;
    const uint32_t hk = r.second ? h - hp.heads0 : h;
    r.ri = r.second ? t * (hp.heads - hp.heads0) + hk : t * hp.heads0 + hk;
    r.ri0 = 0;
    r.xoff = (uint64_t)t * (r.second ? hp.xs1 : hp.xs0) + (uint64_t)hk * D;
  }
  r.trow = r.tok;
  if constexpr (POS && !MT) {
    // positions outside [0, max_pos) read the last table row (never out of range)
    if constexpr (ALIGNED) {
      // a wave-uniform index: read it through the constant address space (the
      // kernel never writes positions), which gives a scalar load; a vector
      // load would make the first use of its value wait for every earlier
      // vector access, the previous pass's stores included
      typedef const __attribute__((address_space(4))) int32_t const_i32;
      const int32_t v = ((const_i32*)p.positions)[r.tok];
      r.trow = __builtin_amdgcn_readfirstlane(min((uint32_t)v, p.max_pos - 1));
    } else {
      r.trow = min((uint32_t)p.positions[r.tok], p.max_pos - 1);
    }
  }
  return r;
}

template <class DT, int L, int MODE, bool ALIGNED, bool MT = false>
__global__ __launch_bounds__(RT) void rows_kernel(const uint16_t* x0, uint64_t x1_or_mt, uint64_t xs0, uint64_t xs1,
                                                   uint32_t waves, uint32_t passes, uint32_t heads, uint32_t heads0,
                                                   uint32_t div_magic, uint32_t shift_rope, RowParams p) {
  const RowHot hp{x0, x1_or_mt, xs0, xs1, waves, passes, heads, heads0, div_magic, shift_rope};
  constexpr bool QUANT = (MODE & ROW_QUANT) != 0;
  constexpr bool ROPE = (MODE & ROW_ROPE) != 0;
  constexpr bool WY = (MODE & ROW_Y) != 0;
  constexpr bool WR = (MODE & ROW_RSTD) != 0;
  constexpr bool POS = (MODE & ROW_POS) != 0;
  constexpr int D = 16 * L;
  constexpr int G = 64 / L;
  // each wave stages its own copy of both tensors' weights (fp32): no
  // workgroup barrier, so a wave starts on its first pass as soon as that
  // pass's input has arrived (a barrier made every wave wait for the slowest
  // first input of its workgroup)
  __shared__ float w_lds[RW * 2 * D];
  // passes inside one token: each wave stages the token's cos and sin rows
  // here (every row of the pass uses the same row); on passes of whole tokens
  // every row has a token of its own and its rope lanes load their values
  // directly, with the pass's input (DIRECT)
  constexpr bool STAGED = ALIGNED && ROPE && !MT;
  constexpr bool DIRECT = MT && ROPE;
  constexpr int TW = D;  // floats per wave
  __shared__ float t_lds[STAGED ? RW * TW : 1];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t u = lane % L;
  float* const w_wave = w_lds + wave * (2 * D);
  const uint32_t slot = lane / L;

  // XCD-aware renumbering: hardware places workgroup b on XCD b % 8; give the
  // workgroups of one XCD a contiguous stretch of the wave numbers.
  // (a select, not a branch: the compiler issues no kernel-argument load past
  // a branch, so a branch here made the argument loads two dependent rounds,
  // each a full memory latency before the first input load goes out)
  uint32_t blk = blockIdx.x;
  {
    // (the grid's size from the preloaded wave count: the grid size itself is
    // a kernel argument the hardware does not preload)
    const uint32_t nb = (hp.waves + RW - 1) / RW, full = nb & ~7u;
    const uint32_t moved = (blk & 7u) * (full >> 3) + (blk >> 3);
    blk = blk < full ? moved : blk;
  }
  const uint32_t gw = blk * RW + wave;
  const uint32_t W = hp.waves, n = p.per_wave, last = hp.passes - 1;
  // (waves past p.waves, at most RW - 1 in the last workgroup, repeat passes of
  // other waves, clamped into range, and write identical bytes: an early exit
  // would be a branch ahead of the kernel-argument loads, see below)
#if RNQ_ROWS_CHUNKED
  auto pass_of = [&](uint32_t i) { return min(gw * n + i, last); };
#else
  auto pass_of = [&](uint32_t i) { return min(gw + i * W, last); };
#endif

  // ---- this lane's columns
  const uint32_t R = ROPE ? hp.rope() : 0u, half = R / 2;
  const uint32_t n_plain = (D - R) / 16;  // units outside the rope tail
  const bool rope_lane = u >= n_plain;
  // (selects, not an if / else: no branch ahead of the kernel-argument loads,
  // see the renumbering below)
  const uint32_t j_tail = u - n_plain;  // (used on rope lanes only)
  const uint32_t off_a = rope_lane ? (D - R) + 8 * j_tail : 16 * u;
  const uint32_t off_b = rope_lane ? off_a + half : off_a + 8;
  const uint32_t cs_off = rope_lane ? 8 * j_tail : 0u;
  // aligned passes: element offsets of this lane's chunks from the pass's first row
  // (outputs: contiguous rows; inputs: tokens xs0 elements apart when a pass holds
  // several tokens, the row's place inside its token otherwise)
  const uint32_t pe_a = slot * D + off_a, pe_b = slot * D + off_b;
  uint32_t px0 = slot * D;
  if constexpr (MT) px0 = (slot >> hp.tok_shift()) * hp.mt_xs() + (slot & ((1u << hp.tok_shift()) - 1u)) * D;
  const uint32_t px_a = px0 + off_a, px_b = px0 + off_b;
  // passes inside one token: lane l carries bytes [TB l, TB l + TB) of the
  // token's cos row and of its sin row (half <= D / 2 floats: 64 lanes of TB
  // bytes cover it, each byte read once; lanes past the row read zero)
  constexpr uint32_t TB = D / 32 < 4 ? 4u : (uint32_t)(D / 32);
  const uint32_t toff = TB * lane;
  // the pass's table block: one row, or the rows of its tokens in order
  const uint32_t tpp = MT ? (uint32_t)G >> hp.tok_shift() : 1u;  // tokens per pass
  const uint32_t tbytes = 4u * half * tpp;                      // bytes of the block (cos or sin)
  // passes of whole tokens: bytes a pass's input rows span (below 2^31, checked
  // by the launcher)
  const uint32_t mt_span = MT ? 2u * ((tpp - 1u) * hp.mt_xs() + (1u << hp.tok_shift()) * (uint32_t)D) : 0u;
  const bool t_lane = toff < tbytes;
  float* t_wave = t_lds + (STAGED ? wave * TW : 0);
  // (passes of whole tokens: from the preloaded arguments)
  const float* const cos_tab = MT ? hp.mt_cos() : p.cos;
  const float* const sin_tab = MT ? hp.mt_sin() : p.sin;

  auto load_staged_table = [&](Data& d) {
    const rsrc_t rc = make_rsrc(cos_tab + (size_t)d.loc.trow * half, tbytes);
    const rsrc_t rs = make_rsrc(sin_tab + (size_t)d.loc.trow * half, tbytes);
    if constexpr (TB == 4) {
      d.cw.x = buf_load4(rc, toff);
      d.sw.x = buf_load4(rs, toff);
    } else if constexpr (TB == 8) {
      const uint2 c = buf_load8(rc, toff), s2 = buf_load8(rs, toff);
      d.cw.x = c.x, d.cw.y = c.y, d.sw.x = s2.x, d.sw.y = s2.y;
    } else {
      d.cw = buf_load16(rc, toff);
      d.sw = buf_load16(rs, toff);
    }
  };
  // passes of whole tokens: a rope lane's 8 cos and 8 sin values, from its
  // row's token (the pass's tokens are consecutive table rows); plain lanes
  // read outside the block (zero, no memory access)
  // (with positions: the row its token's position names, clamped into the
  // table, whose bytes stay below 2^31, checked by the launcher)
  auto load_direct_table = [&](Data& d) {
    rsrc_t rc, rs;
    uint32_t o;
    if constexpr (POS) {
      const uint32_t trow = min(d.pos, p.max_pos - 1u);
      rc = make_rsrc(cos_tab, 4u * p.max_pos * half);
      rs = make_rsrc(sin_tab, 4u * p.max_pos * half);
      o = rope_lane ? 4u * (trow * half + cs_off) : 0x80000000u;
    } else {
      rc = make_rsrc(cos_tab + (size_t)d.loc.trow * half, tbytes);
      rs = make_rsrc(sin_tab + (size_t)d.loc.trow * half, tbytes);
      o = rope_lane ? 4u * ((slot >> hp.tok_shift()) * half + cs_off) : 0x80000000u;
    }
    d.tab.c0 = buf_load16f(rc, o);
    d.tab.c1 = buf_load16f(rc, o + 16u);
    d.tab.s0 = buf_load16f(rs, o);
    d.tab.s1 = buf_load16f(rs, o + 16u);
  };
  // a pass's input (and, through load_data, its table chunks)
  auto load_input = [&](Data& d, uint32_t pass) {
    d.loc = locate<G, D, ALIGNED, POS, MT>(p, hp, pass, slot);
    if constexpr (MT && POS) {
      // this lane's token's position, before the input: the wait for it (ahead
      // of the table loads) then leaves the input in flight
      const rsrc_t rp = make_rsrc(hp.mt_pos(), 4u * ((hp.passes * (uint32_t)G) >> hp.tok_shift()));
      d.pos = buf_load4(rp, 4u * (d.loc.tok + (slot >> hp.tok_shift())));
    }
    if constexpr (ALIGNED) {
      // the pass's G rows: one wave-uniform descriptor, lane byte offsets
      const rsrc_t rx = make_rsrc((d.loc.second && !MT ? hp.x1() : hp.x0) + d.loc.xoff, MT ? mt_span : 2u * G * D);
      d.xa = buf_load16_nt(rx, 2u * px_a);
      d.xb = buf_load16_nt(rx, 2u * px_b);
    } else {
      const uint16_t* src = (d.loc.second ? hp.x1() : hp.x0) + d.loc.xoff;
      d.xa = load_stream16(src + off_a);
      d.xb = load_stream16(src + off_b);
    }
  };
  auto load_data = [&](Data& d, uint32_t pass) {
    load_input(d, pass);
    // the token's cos and sin rows (wave-uniform descriptors), one chunk of
    // each per lane, in flight with the input: the wait for a pass's input
    // covers them, and it never waits on the previous pass's stores. (With a
    // positions index the row number is itself a load: the table chunks then
    // go out from the middle of the previous pass, see compute.)
    if constexpr (STAGED && !POS) load_staged_table(d);
    if constexpr (DIRECT && !POS) load_direct_table(d);
  };
  // per-lane rows: every lane loads its own table values (plain lanes read the
  // row start and ignore it); aligned rope passes load theirs with the input
  auto load_table = [&](Table& t, const Loc& r) {
    if constexpr (ROPE) {
      if constexpr (ALIGNED) {
      } else {
        const float* cp = p.cos + (size_t)r.trow * half + cs_off;
        const float* sp = p.sin + (size_t)r.trow * half + cs_off;
        t.c0 = *(const float4*)cp;
        t.c1 = *(const float4*)(cp + 4);
        t.s0 = *(const float4*)sp;
        t.s1 = *(const float4*)(sp + 4);
      }
    }
  };

  // t: this pass's table values; aligned rope passes stage them in LDS and
  // then load the next pass's table (at `next`) into t.
  // nd: the next pass's data (positions mode: its table chunks are loaded here)
  // nxt: whether a next pass follows (a std::integral_constant<bool>); with
  // positions its table loads go out from the middle of this pass
  auto compute = [&](const Data& s, Table& t, Data& nd, auto opts, auto nxt) {
    constexpr bool NEXT = decltype(nxt)::value;
    constexpr bool GEN = decltype(opts)::gen;
    constexpr bool FULL = decltype(opts)::full;  // the rope tail is the whole row: every lane rotates
    constexpr bool XCH = decltype(opts)::xch;
    const Loc& r = s.loc;
    const float* w = w_wave + (r.second ? D : 0);

    // ---- sum of squares: fp64 (exact for 16-bit inputs), reduced over the row's lanes
    float xv[16];
    unpack8<DT>(s.xa, xv);
    unpack8<DT>(s.xb, xv + 8);
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc = __builtin_fma((double)xv[e], (double)xv[e], acc);
    acc = group_sum<L>(acc);
    const float ssq = (float)acc;               // one rounding of the exact sum
    const float ms = ssq * (1.0f / (float)D);   // D is a power of two: equals ssq / D
    const float rstd = rstd_of(ms + p.eps);

    // ---- normalise: (x * rstd) * w, rounded to the input dtype (values kept as fp32)
    const float4 wa0 = *(const float4*)(w + off_a), wa1 = *(const float4*)(w + off_a + 4);
    const float4 wb0 = *(const float4*)(w + off_b), wb1 = *(const float4*)(w + off_b + 4);
    const float wv[16] = {wa0.x, wa0.y, wa0.z, wa0.w, wa1.x, wa1.y, wa1.z, wa1.w,
                          wb0.x, wb0.y, wb0.z, wb0.w, wb1.x, wb1.y, wb1.z, wb1.w};
    // (fp16 outputs that are only stored stay as fp16 bits: h)
    constexpr bool H16 = __is_same(DT, F16) && !QUANT;
    float y[16];
    uint32_t h[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (H16)
        h[e] = f16_bits((xv[e] * rstd) * wv[e]);
      else
        y[e] = DT::round((xv[e] * rstd) * wv[e]);
    }

    // positions mode: the next pass's table chunks, now that its row number
    // (a scalar load issued with its input) has arrived; still before this
    // pass's stores
    if constexpr (STAGED && POS && NEXT) load_staged_table(nd);
    if constexpr (DIRECT && POS && NEXT) load_direct_table(nd);

    if constexpr (STAGED) {
      // this pass's cos and sin rows into the wave's LDS slot; a wave's LDS
      // accesses complete in order, so the reads below see these writes and the
      // previous pass's reads are done before they land
      // (the cos row, then the sin row: half floats each)
      const uint32_t sin_at = half;
      if (t_lane) {
        if constexpr (TB == 4) {
          t_wave[lane] = __uint_as_float(s.cw.x);
          t_wave[sin_at + lane] = __uint_as_float(s.sw.x);
        } else if constexpr (TB == 8) {
          *(uint2*)(t_wave + 2 * lane) = make_uint2(s.cw.x, s.cw.y);
          *(uint2*)(t_wave + sin_at + 2 * lane) = make_uint2(s.sw.x, s.sw.y);
        } else {
          *(uint4*)(t_wave + 4 * lane) = s.cw;
          *(uint4*)(t_wave + sin_at + 4 * lane) = s.sw;
        }
      }
    }

    // ---- RoPE on the tail: lo' = lo c - hi s, hi' = hi c + lo s, each rounded to dtype
    if constexpr (ROPE) {
      if (FULL || rope_lane) {
        float4 c0 = t.c0, c1 = t.c1, s0 = t.s0, s1 = t.s1;
        if constexpr (DIRECT) {
          c0 = s.tab.c0, c1 = s.tab.c1, s0 = s.tab.s0, s1 = s.tab.s1;
        } else if constexpr (STAGED) {
          const uint32_t sb = half;
          c0 = *(const float4*)(t_wave + cs_off);
          c1 = *(const float4*)(t_wave + cs_off + 4);
          s0 = *(const float4*)(t_wave + sb + cs_off);
          s1 = *(const float4*)(t_wave + sb + cs_off + 4);
        }
        const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float ss[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (H16) {
            const uint32_t lo = h[e], hi = h[8 + e];
            h[e] = f16_bits(mul_f16_f32(lo, cc[e]) - mul_f16_f32(hi, ss[e]));
            h[8 + e] = f16_bits(mul_f16_f32(hi, cc[e]) + mul_f16_f32(lo, ss[e]));
          } else {
            const float lo = y[e], hi = y[8 + e];
            y[e] = DT::round((lo * cc[e]) - (hi * ss[e]));
            y[8 + e] = DT::round((hi * cc[e]) + (lo * ss[e]));
          }
        }
      }
    }

    // element offsets: aligned passes from a wave-uniform row base, else from the tensor start
    const size_t rbase = ALIGNED ? (size_t)r.ri0 * D : (size_t)r.ri * D;
    const uint32_t ea = ALIGNED ? pe_a : off_a, eb = ALIGNED ? pe_b : off_b;
    if constexpr (WY) {
      // the values are already rounded: packing them is exact
      uint16_t* ybase = (r.second ? p.y1 : p.y0) + rbase;
      const uint4 ya = H16 ? pack8_bits(h) : pack8<DT>(y);
      const uint4 yb = H16 ? pack8_bits(h + 8) : pack8<DT>(y + 8);
      if constexpr (ALIGNED) {
        // (nontemporal: path R at 16384 x 128 fp16 4.38 -> 3.97 us against
        // ordinary stores, builds alternated in one process, outputs rotated
        // past the Infinity Cache)
        const rsrc_t ry = make_rsrc(ybase, 2u * G * D);
        buf_store16_nt(ry, 2u * ea, ya);
        buf_store16_nt(ry, 2u * eb, yb);
      } else {
        *(uint4*)((char*)ybase + 2u * ea) = ya;
        *(uint4*)((char*)ybase + 2u * eb) = yb;
      }
    }
    // every lane of the row stores the same value
    if constexpr (WR) p.rstd[r.row] = rstd;

    if constexpr (QUANT) {
      float m = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(y[e]));
      const float amax = group_max_nonneg<L>(m);
      // scale = RN(max(amax, 1e-4) / fp8_max); amax is a 16-bit float value
      float scale;
      if (!GEN || p.scale_by_rcp)
        scale = amax >= 1e-4f ? div_by(amax, p.fp8_max, p.rcp_fp8_max) : p.scale_floor;
      else
        scale = fmaxf(amax, 1e-4f) / p.fp8_max;
      const float rs = rcp_rn(scale);
      float q[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) q[e] = div_by(y[e], scale, rs);
      if (GEN && p.clamp) {
#pragma unroll
        for (int e = 0; e < 16; ++e) q[e] = __builtin_amdgcn_fmed3f(q[e], -p.fp8_max, p.fp8_max);
      }
      uint2 ca, cb;
      ca.x = fp8x4(q[0], q[1], q[2], q[3], __float_as_uint(q[0]));
      ca.y = fp8x4(q[4], q[5], q[6], q[7], __float_as_uint(q[4]));
      cb.x = fp8x4(q[8], q[9], q[10], q[11], __float_as_uint(q[8]));
      cb.y = fp8x4(q[12], q[13], q[14], q[15], __float_as_uint(q[12]));
      uint8_t* cdst = (r.second ? p.c1 : p.c0) + rbase;
      float* sdst = r.second ? p.s1 : p.s0;
      if constexpr (ALIGNED) {
        const rsrc_t rq = make_rsrc(cdst, (uint32_t)(G * D));
        if constexpr (XCH) {
          // whole 16-byte chunks (each store instruction writes whole lines):
          // in a pair of rope lanes (tail chunks 2m and 2m + 1, lanes l and
          // l ^ 1) the even lane keeps its lower-half codes and takes its
          // partner's, the odd lane does the same with the upper half; plain
          // lanes already hold 16 contiguous codes
          // (four DPP moves and four selects per lane; the selects taking the
          // DPP operand directly, through inline assembly, measured no faster)
          const bool odd = (u & 1u) != 0;
          const uint32_t pax = (uint32_t)__builtin_amdgcn_mov_dpp((int)ca.x, 0xB1, 0xF, 0xF, true);
          const uint32_t pay = (uint32_t)__builtin_amdgcn_mov_dpp((int)ca.y, 0xB1, 0xF, 0xF, true);
          const uint32_t pbx = (uint32_t)__builtin_amdgcn_mov_dpp((int)cb.x, 0xB1, 0xF, 0xF, true);
          const uint32_t pby = (uint32_t)__builtin_amdgcn_mov_dpp((int)cb.y, 0xB1, 0xF, 0xF, true);
          const bool rot = FULL || rope_lane;
          const bool lo = !rot || !odd;  // keeps its own first 8 codes
          const bool hi = !rot || odd;   // keeps its own last 8 codes
          const uint4 o = make_uint4(lo ? ca.x : pbx, lo ? ca.y : pby, hi ? cb.x : pax, hi ? cb.y : pay);
          buf_store16_nt(rq, rot && odd ? eb - 8u : ea, o);
        } else {
          buf_store8_nt(rq, ea, ca);
          buf_store8_nt(rq, eb, cb);
        }
        const rsrc_t rsc = make_rsrc(sdst + r.ri0, 4u * G);
        buf_store4(rsc, 4u * slot, scale);  // every lane of the row stores the same value
      } else {
        store_stream8(cdst + ea, ca);
        store_stream8(cdst + eb, cb);
        sdst[r.ri] = scale;
      }
    }
  };

  constexpr int NS = STAGED ? NS_STAGED : 2;  // (two: the register table ring alternates)
  // ---- software pipeline over this wave's n passes: input NS - 1 passes
  // ahead, table values one pass ahead (ring slots are compile-time indices).
  Data d[NS];
  Table tb[2];
  // ---- the first passes' input goes out first: its addresses need only the
  // preloaded arguments. The weights and then the table chunks follow once a
  // load of the kernel arguments has given their pointers; the weights go to
  // LDS after that, and waiting for them waits for the input too (the memory
  // counter is in order), which the first pass needs anyway, but not for the
  // table chunks issued after them. (Scheduling barriers keep this order: the
  // scheduler would otherwise hoist the later loads, and the wait for their
  // pointers, above the input loads.)
#pragma unroll
  for (int k = 0; k < NS - 1; ++k) load_input(d[k], pass_of(k));
  __builtin_amdgcn_sched_barrier(0);
  // weights of both tensors: 16-byte chunks (D / 8 per tensor); lane l loads
  // chunk l % (D / 4) (and l + 64 when D = 512) and stores it in the wave's
  // slot as fp32
  constexpr uint32_t WCH = D / 4;                     // chunks of both tensors
  constexpr uint32_t WPL = WCH > 64 ? WCH / 64 : 1;   // chunks per lane
  uint4 wc[WPL];
#pragma unroll
  for (uint32_t i = 0; i < WPL; ++i) {
    const uint32_t c = (lane + 64 * i) % WCH;
    if constexpr (MT) {
      // (a buffer load: the pointer rebuilt from preloaded integers is generic,
      // and a flat load's wait would also take the table loads and the
      // kernel-argument loads issued after it)
      wc[i] = buf_load16(make_rsrc(hp.mt_w0(), 2u * D), 16u * (c % (D / 8)));
    } else {
      const uint16_t* src = (c < D / 8 ? p.w0 : (hp.heads0 < hp.heads ? p.w1 : p.w0)) + 8 * (c % (D / 8));
      wc[i] = *(const uint4*)src;
    }
  }
  // (the table loads may need kernel-argument fields, such as the table size
  // with positions: kept after the weights, whose loads need none on passes of
  // whole tokens)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (STAGED) {
    // (with positions only the first pass's: each later one goes out from the
    // middle of the pass before it, see compute)
#pragma unroll
    for (int k = 0; k < (POS ? 1 : NS - 1); ++k) load_staged_table(d[k]);
  } else if constexpr (DIRECT) {
    // (with positions only the first pass's, as above)
#pragma unroll
    for (int k = 0; k < (POS ? 1 : NS - 1); ++k) load_direct_table(d[k]);
  } else {
    load_table(tb[0], d[0].loc);
  }
  __builtin_amdgcn_sched_barrier(0);
  // (lanes past the chunks store a copy of the same values: no branch around
  // the loads' use, which would let the compiler sink them under it)
#pragma unroll
  for (uint32_t i = 0; i < WPL; ++i) {
    const uint32_t c = (lane + 64 * i) % WCH;
    float f[8];
    unpack8<DT>(wc[i], f);
    float* dst = w_wave + (c < D / 8 ? 0 : D) + 8 * (c % (D / 8));
    *(float4*)dst = make_float4(f[0], f[1], f[2], f[3]);
    *(float4*)(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
  }

  // Issue priority by progress (launches whose waves are all resident at once):
  // a SIMD's arbiter favours its oldest wave, so the four waves of a SIMD would
  // otherwise finish one after another, the last ones alone on a SIMD whose
  // memory traffic has stopped. Each wave starts at the highest priority and
  // steps down as its share of passes done grows (quarters of n), so waves
  // that are behind issue first and a SIMD's waves finish together.
  const bool by_progress = p.prio_by_progress != 0;
  if (by_progress) __builtin_amdgcn_s_setprio(3);
  auto progress = [&](uint32_t done) {
    if (!by_progress) return;
    const uint32_t q = (4u * done) / n;
    if (q >= 3) __builtin_amdgcn_s_setprio(0);
    else if (q == 2) __builtin_amdgcn_s_setprio(1);
    else if (q == 1) __builtin_amdgcn_s_setprio(2);
  };

  auto run = [&](auto opts) {
    using yes = std::integral_constant<bool, true>;
    uint32_t base = 0;
    for (; base + NS <= n; base += NS) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        load_data(d[(k + NS - 1) % NS], pass_of(base + k + NS - 1));
        if constexpr (STAGED || DIRECT) {
          compute(d[k], tb[0], d[(k + 1) % NS], opts, yes{});
        } else {
          load_table(tb[(k + 1) % 2], d[(k + 1) % NS].loc);
          compute(d[k], tb[k % 2], d[k], opts, yes{});
        }
        progress(base + k + 1);
      }
    }
    // the last n % NS passes: their input (slots 0 .. NS - 2) and first table
    // are loaded; the final one has no next pass (with positions it loads no
    // further table rows)
    auto tail = [&](auto self, auto kc) -> void {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < NS - 1) {
        constexpr bool has_next = k + 1 < NS - 1;
        if (base + k < n) {
          if constexpr (STAGED || DIRECT) {
            compute(d[k], tb[0], d[has_next ? k + 1 : k], opts, std::integral_constant<bool, has_next>{});
          } else {
            if constexpr (has_next) load_table(tb[(k + 1) % 2], d[k + 1].loc);
            compute(d[k], tb[k % 2], d[k], opts, std::integral_constant<bool, has_next>{});
          }
        }
        self(self, std::integral_constant<int, k + 1>{});
      }
    };
    tail(tail, std::integral_constant<int, 0>{});
  };
  // (XCH only where codes are stored from a wave-uniform base, to 16-byte aligned outputs)
  constexpr bool XQ = QUANT && ALIGNED;
  const bool xch = XQ && p.code16 != 0;
  if (QUANT && (p.clamp || !p.scale_by_rcp))
    run(Opts<true, false>{});
  else if (ROPE && R == (uint32_t)D && xch)
    run(Opts<false, true, XQ>{});
  else if (ROPE && R == (uint32_t)D)
    run(Opts<false, true>{});
  else if (xch && (D - R) % 32u == 0 && R % 32u == 0)
    run(Opts<false, false, XQ>{});
  else
    run(Opts<false, false>{});
}

// (how a launch's passes sit in the rows: RowsAlign, rnq_launch.h)

template <int MODE>
hipError_t launch_rows_mode(const RowParams& p, int head_dim, bool bf16, int align, dim3 grid, hipStream_t s);

}  // namespace rnq
