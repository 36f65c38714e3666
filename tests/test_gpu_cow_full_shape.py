"""Copy-on-write at the full shape of the shared-prefix sampling workload
(64 prompts x 8 samples, 40 heads, head_dim 128, bf16, 16-token blocks,
1000-token prompts, tails uniform in [1, 512]), the way a server builds it
("pagedattention vllm" glossary, Copy-on-Write Sharing: Prefix Sharing,
Reference Counting, Divergence Handling):

* the C++ block manager prefills every prompt, forks it for the samples and
  appends their tokens one decode step at a time; its tables, slots and copy
  pairs must equal the oracle twin's bit for bit (448 pairs: 7 per prompt,
  sample 7 writing in place);
* on the GPU the library stores every token, pkv_copy_blocks makes the
  copies the tables name at the divergence step (before any sample token
  lands in them), and the decode step attends through those tables, with the
  plain per-sample call and with the shared-prefix call;
* the oracle replays the same stores and copies on a host pool holding the
  blocks of three prompts (24 sequences: the samples that copied and the one
  that wrote in place), from values it generates itself, and its attention
  for those sequences is the reference.  No value the library computed
  reaches the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_339_amd as pkv
from synthetic import CONFIGS, POISON_BITS, make_layout, shared_prefix_groups, to_storage
from tests.cow_replay import check_divergence_structure, replay_shared_prefix
from tests.gpu_util import assert_rows_close, ints, record_error, say, to_device, widen

pytestmark = pytest.mark.gpu

SELECTED = (0, 31, 63)          # prompts whose values the oracle replays


def _host_values(seed, p, shape):
    """N(0, 1) values of prompt p's tokens, drawn on the host, bf16 bits."""
    return to_storage(np.random.default_rng([seed, 1000 + p]).standard_normal(shape), "bf16")


def test_shared_prefix_copy_on_write_full_shape():
    cfg = CONFIGS[5]
    lay = make_layout(cfg, seed=5)
    S, spp, P, B = len(lay.context_lens), cfg.samples_per_prompt, cfg.prompt_len, cfg.block_size
    Hq, Hkv, D, N = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, lay.num_blocks
    n_prompts = S // spp
    tails = lay.context_lens.astype(np.int64) - P
    T = int(tails.max())
    say(f"cow full shape: {n_prompts} prompts x {spp} samples, pool {N} blocks, tails up to {T}")

    # --- control plane: C++ block manager and the oracle twin, same policy ---
    rep = replay_shared_prefix(cfg, lay)
    check_divergence_structure(cfg, rep)
    prompt_slots, step_slots, div_pairs, tables, lens = (rep.prompt_slots, rep.step_slots, rep.div_pairs,
                                                         rep.tables, rep.lens)
    assert np.array_equal(lens, lay.context_lens)
    say(f"cow full shape: block manager == twin, {len(div_pairs)} copy pairs")

    # --- values: host-drawn for the selected prompts, device-drawn for the rest ---
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(505)

    def dev_randn(*shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    sel_seqs = [p * spp + k for p in SELECTED for k in range(spp)]
    host_prompt = {p: (_host_values(5, p, (P, Hkv, D)), _host_values(6, p, (P, Hkv, D))) for p in SELECTED}
    host_tail = {s: (_host_values(7, s, (int(tails[s]), Hkv, D)), _host_values(8, s, (int(tails[s]), Hkv, D)))
                 for s in sel_seqs}
    q_host = to_storage(np.random.default_rng([5, 1]).standard_normal((S, Hq, D)), "bf16")

    # --- GPU: prompts stored, copies at the divergence step, tails stored ---
    poison = torch.full((N, Hkv, B, D), -1, dtype=torch.int16, device=dev)
    kc, vc = poison.view(torch.bfloat16), poison.clone().view(torch.bfloat16)
    pk, pv = dev_randn(n_prompts, P, Hkv, D), dev_randn(n_prompts, P, Hkv, D)
    for p in SELECTED:
        pk[p] = to_device(host_prompt[p][0], "bf16")
        pv[p] = to_device(host_prompt[p][1], "bf16")
    pkv.reshape_and_cache(pk.view(-1, Hkv, D), pv.view(-1, Hkv, D), kc, vc, ints(np.concatenate(prompt_slots)))
    pkv.copy_blocks(kc, vc, ints(div_pairs))
    rows_seq, rows_t, rows_slot = [], [], []
    last = np.full(S, -1, dtype=np.int32)
    for t, (seqs, sl) in enumerate(step_slots):
        fin = tails[seqs] == t + 1
        last[seqs[fin]] = sl[fin]
        rows_seq.append(seqs[~fin])
        rows_t.append(np.full(int((~fin).sum()), t))
        rows_slot.append(sl[~fin])
    rows_seq, rows_t, rows_slot = np.concatenate(rows_seq), np.concatenate(rows_t), np.concatenate(rows_slot)
    tk, tv = dev_randn(len(rows_seq), Hkv, D), dev_randn(len(rows_seq), Hkv, D)
    pick = np.nonzero(np.isin(rows_seq, sel_seqs))[0]
    hk = np.stack([host_tail[int(rows_seq[i])][0][rows_t[i]] for i in pick])
    hv = np.stack([host_tail[int(rows_seq[i])][1][rows_t[i]] for i in pick])
    idx = torch.from_numpy(pick).to(dev)
    tk.index_copy_(0, idx, to_device(hk, "bf16"))
    tv.index_copy_(0, idx, to_device(hv, "bf16"))
    pkv.reshape_and_cache(tk, tv, kc, vc, ints(rows_slot))
    kn, vn = dev_randn(S, Hkv, D), dev_randn(S, Hkv, D)
    for s in sel_seqs:
        kn[s] = to_device(host_tail[s][0][-1], "bf16")
        vn[s] = to_device(host_tail[s][1][-1], "bf16")
    q = to_device(q_host, "bf16")
    dt, dl, dslots = ints(tables), ints(lens), ints(last)
    max_ctx = int(lens.max())

    # The step as a server runs it: the last token stored and attention, per
    # sample (plain call, cache-resident re-reads of the shared prompt) ...
    out_a = torch.empty_like(q)
    pkv.decode_step(out_a, q, kn, vn, kc, vc, dslots, dt, dl, cfg.scale, B, Hkv, max_ctx,
                    partition_size=cfg.partition_size, cache_policy=cfg.cache_policy)
    # ... and with each prompt's shared blocks read once for its samples.
    members, prefix = shared_prefix_groups(lay)
    out_b = torch.empty_like(q)
    pkv.reshape_and_cache(kn, vn, kc, vc, dslots)
    pkv.paged_attention_decode_shared_prefix(out_b, q, kc, vc, dt, dl, ints(prefix), ints(members),
                                             int(prefix.max()), cfg.scale, B, Hkv, max_ctx)
    torch.cuda.synchronize()

    # --- oracle: the same stores and copies on the selected prompts' blocks ---
    blocks = sorted({int(b) for s in sel_seqs for b in tables[s] if b >= 0})
    remap = {b: i for i, b in enumerate(blocks)}
    hk_c = np.full((len(blocks), Hkv, B, D), POISON_BITS["bf16"], dtype=np.uint16)
    hv_c = hk_c.copy()

    def mapped(slots):
        return np.array([remap[int(x) // B] * B + int(x) % B for x in slots], dtype=np.int64)

    for p in SELECTED:
        oracle.reshape_and_cache(host_prompt[p][0], host_prompt[p][1], hk_c, hv_c, mapped(prompt_slots[p]), B)
    sel_pairs = [(remap[int(a)], remap[int(b)]) for a, b in div_pairs if int(a) in remap]
    assert len(sel_pairs) == len(SELECTED) * (spp - 1)
    oracle.copy_blocks(hk_c, hv_c, sel_pairs)
    for i in pick:
        s, t = int(rows_seq[i]), int(rows_t[i])
        oracle.reshape_and_cache(host_tail[s][0][t:t + 1], host_tail[s][1][t:t + 1], hk_c, hv_c,
                                 mapped([rows_slot[i]]), B)
    for s in sel_seqs:
        oracle.reshape_and_cache(host_tail[s][0][-1:], host_tail[s][1][-1:], hk_c, hv_c, mapped([last[s]]), B)
    sel_tables = np.array([[remap[int(b)] if b >= 0 else -1 for b in tables[s]] for s in sel_seqs])
    want = oracle.paged_attention_decode(q_host[sel_seqs], hk_c, hv_c, sel_tables, lens[sel_seqs], cfg.scale, B,
                                         Hkv, "bf16")

    sel = torch.tensor(sel_seqs, device=dev)
    err_a = assert_rows_close(widen(out_a.index_select(0, sel)), want, "bf16", "cow full shape, per-sample call")
    err_b = assert_rows_close(widen(out_b.index_select(0, sel)), want, "bf16", "cow full shape, shared-prefix call")
    say(f"cow full shape: sequences {sel_seqs[0]}..{sel_seqs[-1]} (3 prompts), max row-relative error "
        f"{err_a:.2e} (per-sample call), {err_b:.2e} (shared-prefix call)")
    record_error("cow_full_shape/per_sample_call", err_a, sequences=sel_seqs)
    record_error("cow_full_shape/shared_prefix_call", err_b, sequences=sel_seqs)
