"""Block-sparse masked attention for AMD Instinct MI355X (gfx950).

The public functions live in `api` and load the HIP library libbsm.so on
first use; importing the package alone does not, so that `build` can run
before the library exists.  There is no fallback: a missing library raises
ImportError.
"""
_API_NAMES = {"MaskSpec", "MaskTerm", "CAUSAL", "SAME_DOC", "IN_WINDOW", "SINK", "PREFIX",
              "and_masks", "or_masks", "ScoreMod", "BlockMask", "mask_spec", "from_spec_data", "score_mod",
              "empty_block_mask", "build_block_mask", "flex_attention_fwd",
              "flex_attention_bwd", "bwd_workspace", "block_mask_workspace",
              "flex_attention_decode", "flex_attention_decode_static", "flex_attention_decode_paged",
              "gather_kv_pages", "flex_attention_decode_multi_paged",
              "decode_workspace",
              "decode_multi_spec", "flex_attention_decode_multi"}


def __getattr__(name):
    if name in _API_NAMES:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)


__all__ = sorted(_API_NAMES)
