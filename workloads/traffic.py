"""Seeded synthetic request streams with the reuse structures the pages
describe for prefix caching ([P2] "What reuse is worth": few-shot
classification, agent loop, multi-turn chat, RAG question answering).

Only token ids and request structure are drawn here (no allocator logic, no
matching): each request is a prompt, and for chat and agent traffic the
continuation the model "generated" (random ids) that the next request of the
same session resends.  Sizes:

* few_shot: a 1,900-token block of examples shared by every request, then a
  100-token item under test (95% of the prompt shared).
* agent: 1,800 tokens of tool schemas and instructions, then a scratchpad
  that grows by one 200-token step per call; every call resends everything.
* chat: a 300-token system prompt, then turns of a 60-token user message and
  a 120-token reply; turn k resends the whole conversation.
* rag: a 150-token system prompt, 1,500 tokens of retrieved passages that
  differ per query, and a 30-token question.

Each stream has ``sessions`` independent sessions (distinct random tails);
all share the same system-level prefix.
"""

from __future__ import annotations

import random
from dataclasses import dataclass, field

VOCAB = 32000


@dataclass
class Request:
    session: int
    prompt: list
    reply: list = field(default_factory=list)  # ids generated after the prompt (kept in the cache)


def _ids(rng: random.Random, n: int) -> list:
    return [rng.randrange(VOCAB) for _ in range(n)]


def few_shot(seed: int = 1, requests: int = 64) -> list:
    rng = random.Random(seed)
    examples = _ids(rng, 1900)
    return [Request(i, examples + _ids(rng, 100)) for i in range(requests)]


def agent(seed: int = 2, sessions: int = 4, steps: int = 12) -> list:
    rng = random.Random(seed)
    tools = _ids(rng, 1800)
    out = []
    pads = {s: [] for s in range(sessions)}
    for step in range(steps):
        for s in range(sessions):
            pads[s] = pads[s] + _ids(rng, 200)
            out.append(Request(s, tools + list(pads[s]), reply=_ids(rng, 40)))
            pads[s] = pads[s] + out[-1].reply
    return out


def chat(seed: int = 3, sessions: int = 4, turns: int = 8) -> list:
    rng = random.Random(seed)
    system = _ids(rng, 300)
    conv = {s: list(system) for s in range(sessions)}
    out = []
    for turn in range(turns):
        for s in range(sessions):
            conv[s] = conv[s] + _ids(rng, 60)
            r = Request(s, list(conv[s]), reply=_ids(rng, 120))
            out.append(r)
            conv[s] = conv[s] + r.reply
    return out


def rag(seed: int = 4, requests: int = 64) -> list:
    rng = random.Random(seed)
    system = _ids(rng, 150)
    return [Request(i, system + _ids(rng, 1500) + _ids(rng, 30)) for i in range(requests)]


STREAMS = {"few_shot": few_shot, "agent": agent, "chat": chat, "rag": rag}
