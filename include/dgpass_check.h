/*
 * dgpass_check.h -- host-only self-checks of libdgpass's launch plans.
 *
 * No device work: these replay, on the CPU, the arithmetic a kernel uses to
 * form its memory addresses, so that a test can show every access stays in
 * bounds for shapes no device run has covered.
 */
#ifndef DGPASS_CHECK_H
#define DGPASS_CHECK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The attention of a denoising pass (mode 0) or of a prefill (mode 1), with
 * activations of storage type act_dtype (DG_F32 or DG_BF16: the two use
 * different kernels and tile schedules), over B
 * requests of T new rows each, with len[b] cached keys (host array [B]), Hq
 * query heads sharing Hkv key/value heads and room for part_cap (row, head)
 * entries of key-split partials.  Course page "Module 12. Diffusion Language
 * Models", block-mask exercise: every query of the active block reads the
 * complete prefix and block of its own request (prefix rows are causal).
 * Replays the launch plan, the block decode and the key index of every staged
 * K/V slot, and returns how many of those slots address a key that is not one
 * of the block's own request (mode 0: cache rows [0, len[b]) and canvas rows
 * [0, T); mode 1: cache rows [0, len[b] + T)), plus one if the partials
 * would overflow part_cap; 0 means every access is in bounds.  *nslots (may
 * be NULL) receives the number of slots checked.  Returns -1 for invalid
 * arguments (B outside [1, DG_MAX_BATCH], T < 1, Hq not a multiple of Hkv,
 * another act_dtype). */
long dg_check_attention_addresses(int act_dtype, int B, int T, const int32_t* len, int Hq, int Hkv,
                                  int mode, long part_cap, long* nslots);

#ifdef __cplusplus
}
#endif
#endif
