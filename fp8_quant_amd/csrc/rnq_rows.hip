// Row-kernel launcher: host-side set-up shared by every mode (the kernel is
// in rnq_rows.h; its modes are instantiated in rnq_rows_quant.hip and
// rnq_rows_norm.hip).
#include "rnq_rows.h"

namespace rnq {

#ifndef RNQ_ROWS_TARGET_WAVES
#define RNQ_ROWS_TARGET_WAVES 4096  // 4 per SIMD: what stays resident at the kernel's register use
#endif
#ifndef RNQ_ROWS_PRIO
#define RNQ_ROWS_PRIO 1  // issue priority by progress: 0 never, 1 when every wave is resident at once, 2 always
#endif
#ifndef RNQ_ROWS_MAX_PER_WAVE
#define RNQ_ROWS_MAX_PER_WAVE 8  // larger launches: more waves, dispatched in order as others retire
#endif

hipError_t launch_rows(RowParams p, int head_dim, bool bf16, bool quant, hipStream_t stream) {
  if (p.total_rows == 0) return hipSuccess;
  const uint32_t G = 64u / (uint32_t)(head_dim / 16);
  p.passes = (uint32_t)((p.total_rows + G - 1) / G);
  // t = row / heads by multiply-shift (exact for every row < 2^31)
  div_magic_for(p.heads, p.div_magic, p.div_shift);
  // the same number of passes for every wave: as few waves as keep the
  // SIMDs busy, at most RNQ_ROWS_MAX_PER_WAVE passes each. Waves that do not
  // fit at once start as others retire, in launch order, so the active
  // passes stay within a narrow window of the tensors.
  p.per_wave = (p.passes + RNQ_ROWS_TARGET_WAVES - 1) / RNQ_ROWS_TARGET_WAVES;
  if (p.per_wave > RNQ_ROWS_MAX_PER_WAVE) p.per_wave = RNQ_ROWS_MAX_PER_WAVE;
  p.waves = (p.passes + p.per_wave - 1) / p.per_wave;
  // (more waves than stay resident start as earlier ones retire, oldest first:
  // progress priority only where they all run at once)
  p.prio_by_progress = RNQ_ROWS_PRIO == 2 || (RNQ_ROWS_PRIO == 1 && p.per_wave > 1 && p.waves <= RNQ_ROWS_TARGET_WAVES)
                           ? 1u : 0u;
  const dim3 grid((p.waves + RW - 1) / RW);
  // scale = RN(max(amax, 1e-4) / fp8_max) through the reciprocal of fp8_max
  // when fp8_max >= 1 (no overflow for any 16-bit amax)
  p.rcp_fp8_max = 1.0f / p.fp8_max;
  p.scale_floor = 1e-4f / p.fp8_max;
  p.scale_by_rcp = p.fp8_max >= 1.0f ? 1u : 0u;
  p.clamp = quant && fp8_clamp_needed(p.fp8_max) ? 1u : 0u;
  // (the entry points accept 8-byte aligned code outputs; 16-byte code stores need 16)
  p.code16 = ((uintptr_t)p.c0 % 16 == 0 && (uintptr_t)p.c1 % 16 == 0) ? 1u : 0u;
  // contiguous inputs unless the caller gave token strides
  if (p.xs0 == 0) p.xs0 = (uint64_t)p.heads0 * (uint64_t)head_dim;
  if (p.xs1 == 0) p.xs1 = (uint64_t)(p.heads - p.heads0) * (uint64_t)head_dim;
  const bool pos = p.rope > 0 && p.positions != nullptr;
  // passes inside one token and one tensor (both head counts multiples of G,
  // whole passes then), passes of whole tokens of one tensor (their rows at
  // lane-constant offsets, each rope lane reading its own row's table values,
  // with positions at 32-bit offsets into the table), or rows located per lane
  const int align = rows_layout(G, p.heads, p.heads0, p.total_rows, p.xs0, (uint32_t)head_dim, p.rope, pos,
                                p.max_pos, &p.tok_shift);
  const int mode = (quant ? ROW_QUANT : 0) | (p.rope > 0 ? ROW_ROPE : 0) | (p.y0 != nullptr ? ROW_Y : 0) |
                   (p.rstd != nullptr ? ROW_RSTD : 0) | (pos ? ROW_POS : 0);
  switch (mode) {
    case ROW_QUANT: return launch_rows_mode<ROW_QUANT>(p, head_dim, bf16, align, grid, stream);
    case ROW_QUANT | ROW_ROPE: return launch_rows_mode<ROW_QUANT | ROW_ROPE>(p, head_dim, bf16, align, grid, stream);
    case ROW_QUANT | ROW_Y: return launch_rows_mode<ROW_QUANT | ROW_Y>(p, head_dim, bf16, align, grid, stream);
    case ROW_QUANT | ROW_ROPE | ROW_Y:
      return launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_Y>(p, head_dim, bf16, align, grid, stream);
    case ROW_Y: return launch_rows_mode<ROW_Y>(p, head_dim, bf16, align, grid, stream);
    case ROW_Y | ROW_ROPE: return launch_rows_mode<ROW_Y | ROW_ROPE>(p, head_dim, bf16, align, grid, stream);
    case ROW_Y | ROW_RSTD: return launch_rows_mode<ROW_Y | ROW_RSTD>(p, head_dim, bf16, align, grid, stream);
    case ROW_QUANT | ROW_ROPE | ROW_POS:
      return launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_POS>(p, head_dim, bf16, align, grid, stream);
    case ROW_QUANT | ROW_ROPE | ROW_Y | ROW_POS:
      return launch_rows_mode<ROW_QUANT | ROW_ROPE | ROW_Y | ROW_POS>(p, head_dim, bf16, align, grid, stream);
    case ROW_Y | ROW_ROPE | ROW_POS:
      return launch_rows_mode<ROW_Y | ROW_ROPE | ROW_POS>(p, head_dim, bf16, align, grid, stream);
    default: return hipErrorInvalidValue;  // not a combination the entry points produce
  }
}

}  // namespace rnq
