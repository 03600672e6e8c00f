"""Best-of-N selection oracle -- TEST INFRASTRUCTURE ONLY.

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg, like the rest of this package; shares no code with the GPU path.

"Learning to summarize from human feedback" (summary), Method adaptation:
the reward model scores N sampled summaries of a post and the one it scores
highest is kept (best-of-N).  The page does not say how equal rewards are
resolved; the reading used here is the lowest candidate index.

Shared prompts: in a causal (decoder) model a token's state depends only on
the tokens before it, so scoring prompt + candidate gives the same reward
whether the prompt is evaluated once for all its candidates or once per
candidate.  The oracle is the plain definition -- every prompt + candidate
scored as one sequence by OracleModel.score -- and the GPU's shared-prompt
evaluation is checked against it.
"""


def best_of_n(rewards, counts):
    """Index of the best candidate of every prompt.

    rewards: one value per candidate, the candidates of prompt 0 first, then
    those of prompt 1, ...; counts[p] >= 1 candidates belong to prompt p.
    Returns a list with, for every prompt, the index (0-based, within that
    prompt's candidates) of the largest reward; among equal rewards the
    lowest index.
    """
    best = []
    start = 0
    for c in counts:
        c = int(c)
        if c < 1:
            raise ValueError("every prompt needs at least one candidate")
        if start + c > len(rewards):
            raise ValueError("counts ask for more candidates than rewards were given")
        k = 0
        for j in range(1, c):
            if rewards[start + j] > rewards[start + k]:  # strict: an equal later value never wins
                k = j
        best.append(k)
        start += c
    if start != len(rewards):
        raise ValueError("counts do not cover every reward")
    return best
