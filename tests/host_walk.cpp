// Host build of the workgroup -> work-item mappings the kernels use (block_coords,
// ItemWalk, persistent_grid's sizing rule), exported for the bijection test in
// test_grid_mapping.py.  Compiled host-only: nothing here runs on a GPU.
#include "../exact_tiled_attention_12_amd/csrc/attn_common.h"

extern "C" {

// (head, blk) of every workgroup bid < nb of a launch with nblk blocks per head
int walk_block_coords(int causal, int heavy_last, int nb, int nblk, int slots, int* head, int* blk)
{
    for (int b = 0; b < nb; ++b) {
        if (causal && heavy_last) attn::block_coords<true, true>(b, nb, nblk, slots, head[b], blk[b]);
        else if (causal) attn::block_coords<true, false>(b, nb, nblk, slots, head[b], blk[b]);
        else if (heavy_last) attn::block_coords<false, true>(b, nb, nblk, slots, head[b], blk[b]);
        else attn::block_coords<false, false>(b, nb, nblk, slots, head[b], blk[b]);
    }
    return 0;
}

// the items each of nwg persistent workgroups walks, -1 after its share (max_steps per row)
int walk_items(int nwg, int nitems, int nblk, int causal, int max_steps, int* items)
{
    const bool split = causal ? attn::items_split<true>(nitems, nblk) : attn::items_split<false>(nitems, nblk);
    for (int w = 0; w < nwg; ++w) {
        attn::ItemWalk walk;
        walk.init(w, nwg, nitems, split);
        int t = 0;
        for (; t < max_steps; ++t) {
            const int it = walk.item(t);
            items[(long)w * max_steps + t] = it;
            if (it < 0) break;
        }
        if (t == max_steps) return -1;          // a workgroup would walk more than max_steps items
    }
    return 0;
}

// the workgroup count persistent_grid gives for ncu compute units
int persistent_workgroups(int nitems, int per_cu, int split, int ncu)
{
    int n = ncu * per_cu;
    if (n > nitems) n = nitems;
    if (split) n &= ~7;
    if (n < 1) n = 1;
    return n;
}

}  // extern "C"
