"""Plain autoregressive decoding and the DEX lattice (test infrastructure only).

Both drivers take an *evaluator* with the interface of
``oracle.model.SlotEvaluator``: ``begin(prompt)``, ``eval_slots(slots)``,
``logits(slot, depth)``, ``commit(token)`` and the committed length ``C``.

``ar_decode`` is the reference: each step decodes the committed context's
anchor slot at full depth L with the unmodified rule. Alongside each token it
reports what DEX's anchor path would propose at that position (the DECS-masked
candidates u_0..u_{N-1} at depths d_0..d_{N-1}), the branch the commit rule
selects and the brute-force EAD (Definition 1, eqs. (1)-(3)) computed from the
rule's unmasked candidate at every depth 1..L.

``dex_decode`` runs Algorithm 1 of "Depth Exploration for LLM Decoding"
(Section 3.1) on the depth-position lattice of Section 3.2:

* expand - a round turns every node created in the previous round into a
  depth child (same slot, next explorer; none beyond the final explorer) and a
  position child (a new slot whose prefix is extended by the node's candidate,
  starting at explorer 0). The first round of a tree creates the anchor slot's
  explorer-0 node.
* DECS   - every new node decodes its candidate with Algorithm 2.
* commit - once the anchor path reaches the final explorer (the FSM has done
  N rounds since the tree started), the token appended is the final-depth
  candidate u_{N-1}; the selected branch is the shallowest anchor node whose
  candidate equals it, else the final one.
* collapse - only the subtree that continues the committed prefix survives:
  the position child of the selected branch becomes the new anchor slot's
  root; its slots drop the old anchor token; the FSM state becomes the number
  of rounds that subtree has already done (N - 1 - b). With the final branch
  selected nothing survives and a fresh tree starts from the new anchor token.

FSM convention (the paper counts explorer rounds since the last commit and
says state q materialises 2^q - 1 buffer entries): here ``q`` is the number of
rounds the current tree has completed, so the tree holds 2^q - 1 nodes and a
round at state q creates 2^q nodes; the commit happens when q reaches N.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .depth import ead, ead_stable
from .rule import decode


def _gumbel_row(gumbel, target: int, P: int, mode: str):
    if mode != "sample":
        return None
    return gumbel[target - P]


def ar_decode(ev, prompt: Sequence[int], T: int, X: Sequence[int], mode: str = "greedy",
              tau: float = 1.0, gumbel=None, decs: bool = True,
              forced: Optional[Sequence[int]] = None, brute_ead: bool = True,
              keep_logits: bool = False, on_commit=None) -> List[dict]:
    """Plain AR decoding of T tokens; ``gumbel[j]`` is the noise row for target
    position len(prompt) + j. With ``forced`` the context follows the given
    tokens instead of the decoded ones (every reported quantity is still a
    function of the committed prefix only). ``on_commit(record)`` is called
    after each token (progress reporting)."""
    N, L, P = len(X), X[-1], len(prompt)
    ev.begin(list(prompt))
    anchor = int(prompt[-1])
    recs = []
    for t in range(T):
        slot = (anchor,)
        ev.eval_slots([slot])
        g = _gumbel_row(gumbel, ev.C + 1, P, mode)
        z_final = ev.logits(slot, L)
        y, m_final, _ = decode(z_final, [], mode, tau, g)
        u, margins = [], []
        for j in range(N):
            masked = list(u) if (decs and j < N - 1) else []
            uj, mj, _ = decode(ev.logits(slot, X[j]), masked, mode, tau, g)
            u.append(uj)
            margins.append(mj)
        assert u[-1] == y, "final-depth reference must equal the unmasked rule"
        yc = int(forced[t]) if forced is not None else y
        b = next((j for j in range(N) if u[j] == yc), N - 1)
        rec = dict(token=yc, decoded=y, position=ev.C + 1, u=u, margins=margins,
                   b=b, layers=X[b], final_margin=m_final)
        if brute_ead:
            dec = [decode(ev.logits(slot, l), [], mode, tau, g) for l in range(1, L + 1)]
            cand = [d[0] for d in dec]
            acc = [c == yc for c in cand]
            rec.update(cand_by_depth=cand, cand_margins=[d[1] for d in dec], ead=ead(acc),
                       ead_stab=ead_stable(acc))
        if keep_logits:
            rec["final_logits"] = z_final
        recs.append(rec)
        if on_commit is not None:
            on_commit(rec)
        ev.commit(yc)
        anchor = yc
    return recs


@dataclass(eq=False)
class Node:
    etk: int                       # id in the explore buffer (creation order)
    slot: tuple                    # slot tokens, starting with the anchor token
    k: int                         # explorer index; exit depth X[k]
    prior: list                    # shallower nodes of the same slot chain
    round: int
    parent: int = -1               # etk of the node it expanded from
    kind: str = "root"             # "root", "depth" or "position"
    depth_child: Optional["Node"] = None
    pos_child: Optional["Node"] = None
    cand: int = -1
    margin: float = 0.0


def _subtree(n: Node) -> List[Node]:
    out, stack = [], [n]
    while stack:
        x = stack.pop()
        out.append(x)
        for c in (x.depth_child, x.pos_child):
            if c is not None:
                stack.append(c)
    return out


def dex_decode(ev, prompt: Sequence[int], T: int, X: Sequence[int], mode: str = "greedy",
               tau: float = 1.0, gumbel=None, decs: bool = True,
               forced: Optional[Sequence[int]] = None, stats: Optional[dict] = None,
               single_exit: bool = False, branch_cap: int = 0, on_commit=None) -> List[dict]:
    """DEX decoding of T tokens. Returns one record per commit:
    token, b, layers (= d_b), u (anchor candidates), margins, rounds (rounds
    since the previous commit). ``stats`` (optional dict) receives per-round
    node counts per explorer under "rows_per_round". ``on_commit(record)`` is
    called after each commit (progress reporting).

    single_exit: the single-exit ablation of "Depth Exploration for LLM
    Decoding", Section 4 (Figure 4, right-top): intermediate depth branches
    are disabled, so only the first and the final explorer expose candidates.
    Reading: a node of an intermediate explorer is still computed (the chain
    must reach the final depth) but does not exit, so it proposes no token and
    has no position child; the commit keeps branch 0 when u_0 matches and the
    final depth otherwise. Unmasked candidates follow (no shallower proposal
    exists in a chain).

    branch_cap: a pruned lattice (the sparse lattice named as future work in
    Appendix E, "Expansion growth and overhead"). The pages give no policy; the one taken here is structural:
    only nodes of explorers j < branch_cap spawn position children (0: no
    pruning). Depth children are never pruned, so every anchor chain still
    reaches the final depth and the commit rule is unchanged: the output stays
    the plain model's. A commit whose branch b has no position child (b >=
    branch_cap) keeps nothing, and a fresh tree starts from the new anchor,
    as after the final branch."""
    N, P = len(X), len(prompt)
    ev.begin(list(prompt))
    anchor_tok = int(prompt[-1])
    q, root, frontier = 0, None, []
    recs: List[dict] = []
    etk = 0
    rnd = 0
    since = 0
    rows_log, nodes_log = [], []
    while len(recs) < T:
        pruned = 0 < branch_cap < N
        tree = _subtree(root) if root is not None else []
        if not pruned:
            assert len(tree) == (q * (q + 1) // 2 if single_exit else 2 ** q - 1), "nodes held at state q"
        # expand
        if q == 0:
            root = Node(etk=0, slot=(anchor_tok,), k=0, prior=[], round=rnd)
            new = [root]
            etk = 1
        else:
            new = []
            for f in frontier:
                if f.k < N - 1:
                    c = Node(etk=0, slot=f.slot, k=f.k + 1, prior=f.prior + [f], round=rnd,
                             parent=f.etk, kind="depth")
                    f.depth_child = c
                    new.append(c)
                if f.cand is None:
                    continue                           # a node that did not exit
                if pruned and f.k >= branch_cap:
                    continue                           # pruned: no position branch from this explorer
                c = Node(etk=0, slot=f.slot + (f.cand,), k=0, prior=[], round=rnd,
                         parent=f.etk, kind="position")
                f.pos_child = c
                new.append(c)
            for c in new:
                c.etk = etk
                etk += 1
        if single_exit:
            assert len(new) == q + 1, "a single-exit round at state q creates q + 1 nodes"
        elif not pruned:
            assert len(new) == 2 ** q, "a round at state q creates 2^q nodes"
        ev.eval_slots([n.slot for n in new])
        # DECS + insert
        for n in new:
            final = n.k == N - 1
            if single_exit and 0 < n.k < N - 1:
                n.cand, n.margin = None, None
                continue
            masked = [] if (final or not decs) else [p.cand for p in n.prior if p.cand is not None]
            g = _gumbel_row(gumbel, ev.C + len(n.slot), P, mode)
            n.cand, n.margin, _ = decode(ev.logits(n.slot, X[n.k]), masked, mode, tau, g)
        rows_log.append([sum(1 for n in new if n.k == j) for j in range(N)])
        nodes_log.append([(n.etk, n.k, n.parent, n.kind, len(n.slot)) for n in new])
        frontier = new
        rnd += 1
        since += 1
        if q + 1 < N:
            q += 1                                     # advance
            continue
        # ReachFinalDepth: validate and commit
        chain = [root]
        while chain[-1].depth_child is not None:
            chain.append(chain[-1].depth_child)
        assert len(chain) == N and all(c.slot == (anchor_tok,) for c in chain)
        u = [c.cand for c in chain]
        y = u[-1] if forced is None else int(forced[len(recs)])
        b = next((j for j in range(N) if u[j] == y), N - 1)
        recs.append(dict(token=y, decoded=u[-1], position=ev.C + 1, u=u,
                         margins=[c.margin for c in chain], b=b, layers=X[b], rounds=since))
        if on_commit is not None:
            on_commit(recs[-1])
        since = 0
        if len(recs) == T:
            break
        # collapse
        ev.commit(y)
        if b < N - 1 and chain[b].pos_child is not None:
            root = chain[b].pos_child
            assert root.slot == (anchor_tok, y)
            kept = sorted(_subtree(root), key=lambda n: n.etk)
            for i, n in enumerate(kept):        # renumber the surviving buffer
                assert n.slot[:2] == (anchor_tok, y)
                n.slot = n.slot[1:]
                n.etk = i
            etk = len(kept)
            q = N - 1 - b
            frontier = [n for n in kept if n.round == rnd - 1]
        else:
            root, frontier, q = None, [], 0
        anchor_tok = y
    if stats is not None:
        stats["rows_per_round"] = rows_log
        stats["nodes_per_round"] = nodes_log
        stats["rounds"] = rnd
    return recs
