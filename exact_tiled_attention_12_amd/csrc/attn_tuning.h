// Launch parameters per (kernel, head dim, causal, sequence length), chosen by an
// offline sweep on MI355X.  The block sizes of the pages' design are tuned per GPU
// ahead of time and looked up at launch (FlashAttention-2 review, implementation-
// cost answer, section 1 (2), auto-tuning; auto-tuning answer).  The tile shapes of
// these kernels are fixed by their register and LDS budgets; what the sweep picks:
//   slots     -- the causal schedule's L2 group size (block_coords): how many
//                workgroup slots of an XCD one group of heads fills;
//   key_tile  -- keys per tile of the fp8 forward (64 or 128).
// The table below is written by `python -m exact_tiled_attention_12_amd.tune`
// (the measurements it was chosen from are in profiles/tuning_sweep.md); a build
// with ATTN_TUNE_FORCE_SLOTS / ATTN_TUNE_FORCE_KEY_TILE defined ignores it, which
// is how the sweep builds its candidates.
#pragma once

namespace attn {

enum TuneKernel { kTuneFwdBf16 = 0, kTuneFwdF32 = 1, kTuneDkdv = 2, kTuneDq = 3, kTuneFwdFp8 = 4, kTuneBwdF32 = 5 };

struct TuneEntry {
    int kernel, d, causal, n_max;     // an entry applies to N <= n_max (first match in table order)
    int slots, key_tile;
};

// ---- generated table: begin ----
static constexpr TuneEntry kTuneTable[] = {
    {kTuneDkdv, 80, 1, 1 << 30, 32, 64},
    {kTuneDkdv, 128, 1, 4096, 32, 64},
    {kTuneDkdv, 128, 1, 1 << 30, 32, 64},
    {kTuneDq, 80, 1, 1 << 30, 64, 64},
    {kTuneDq, 128, 1, 4096, 128, 64},
    {kTuneDq, 128, 1, 1 << 30, 64, 64},
    {kTuneFwdBf16, 80, 1, 1 << 30, 64, 64},
    {kTuneFwdBf16, 128, 1, 4096, 64, 64},
    {kTuneFwdBf16, 128, 1, 1 << 30, 64, 64},
    {kTuneFwdFp8, 64, 0, 1 << 30, 64, 64},
    {kTuneFwdFp8, 128, 0, 1 << 30, 64, 64},
    {kTuneFwdFp8, 128, 1, 4096, 128, 64},
    {kTuneFwdFp8, 128, 1, 1 << 30, 128, 128},
    {kTuneFwdBf16, 0, 1, 1 << 30, 64, 64},
    {kTuneDkdv, 0, 1, 1 << 30, 32, 64},
    {kTuneDq, 0, 1, 1 << 30, 64, 64},
    {kTuneFwdFp8, 0, 1, 1 << 30, 64, 64},
    {kTuneFwdFp8, 0, 0, 1 << 30, 64, 64},
    {kTuneFwdF32, 0, 1, 1 << 30, 32, 64},
    {kTuneBwdF32, 0, 1, 1 << 30, 32, 64},
};
// ---- generated table: end ----

// d = 0 in an entry matches every head dim.  Unlisted cases: slots 64, key tile 64.
inline TuneEntry tune_lookup(int kernel, int d, int causal, int N)
{
    TuneEntry t{kernel, d, causal, N, 64, 64};
    for (const TuneEntry& e : kTuneTable)
        if (e.kernel == kernel && (e.d == 0 || e.d == d) && e.causal == causal && N <= e.n_max) {
            t = e;
            break;
        }
#ifdef ATTN_TUNE_FORCE_SLOTS
    t.slots = ATTN_TUNE_FORCE_SLOTS;
#endif
#ifdef ATTN_TUNE_FORCE_KEY_TILE
    t.key_tile = ATTN_TUNE_FORCE_KEY_TILE;
#endif
    return t;
}

}  // namespace attn
